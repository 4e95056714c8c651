"""Benchmark of the RAM-Net attention core on one MI355X.

One step = one full pass of the hot path over one batch of synthetic inputs
already resident in HBM: ram_forward (decode both sides, bucket, GSU scan,
read-out) followed by ram_backward (reverse scan, decode backward), at the
1.3B-layer shape: B=8, H=16, T=4096, S=4096 slots per head, top-8 per side,
d_v=128, bf16 io, fp32 state and arithmetic, Zipf(1.1) hot-slot bias.

Prints one JSON line.  ms_per_step comes from K timed steps with nothing
else recorded.  Per-kernel durations come from a second pass of K timed
steps in which the library records HIP events around every launch on the
stream it launches on (ram_prof_*); the roofline of the dominant kernel
(decode_bwd) uses them.  Its HBM traffic comes from the rocprofv3 counter
summary in profiles/ (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the
counts of a copy of known size) and is reported only while the hash of the
kernel's sources matches the one recorded there.  The CPU baseline times the
plain oracle on a bounded sample of (b, h) slices of the same workload on
the host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --config 340m [--flush]   # the 340M layer, caches warm or flushed
  python bench.py --config stream      # HBM read and copy roofs of the decoders' pattern
  python bench.py --copy-calibration   # plain 1 GiB copies (HBM counter scale)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "tokens/sec fwd+bwd per layer on 1 MI355X; achieved HBM GB/s vs peak"


def algorithmic_bytes(cfg, b_io=2):
    """Bytes the method must move per fwd+bwd step: each input read once and
    each output written once per pass (state, logits, values, gradients).
    A logit row holds U * P values (S for one digit)."""
    N = cfg.B * cfg.T * cfg.H
    R, d = cfg.U * cfg.P, cfg.d_v
    nseg = cfg.B * cfg.H * cfg.S
    fwd = N * (2 * R * b_io + d * b_io + b_io + d * b_io) + nseg * (d + 1) * 4
    bwd = N * (2 * R * b_io + 2 * R * b_io + 3 * d * b_io + 2 * b_io)
    return fwd, bwd


def decode_bwd_bytes(cfg, b_io=2):
    """Algorithmic bytes of one decode_bwd launch (both sides): per row the
    U * P logits read and as many gradients written.  The workspace it also
    reads (the U logsumexps and k x (index, weight, weight gradient), 4U + 12k
    bytes per row) is not algorithmic."""
    N = cfg.B * cfg.T * cfg.H
    return 2 * N * 2 * cfg.U * cfg.P * b_io


DECODE_SOURCES = ("linear_attention_ram_amd/csrc/decode.hip", "linear_attention_ram_amd/csrc/decode.hpp",
                  "linear_attention_ram_amd/csrc/decode_prod.hpp",
                  "linear_attention_ram_amd/csrc/common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bwd_1.3b_hbm_traffic.txt")


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode_bwd launch from the committed counter summary, or
    None when it is missing or the decoder sources changed since it was taken."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_hash") != source_hash(DECODE_SOURCES):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, x, threads, budget_s=15.0):
    """Time the oracle's fwd+bwd on (b, h) slices of the workload, `threads`
    slices per call (one per OpenMP thread), until the budget is spent."""
    import numpy as np
    import oracle
    oracle.set_threads(threads)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    done, spent = 0, 0.0
    while done < len(pairs) and spent < budget_s:
        group = pairs[done:done + threads]
        n = len(group)

        def stack(key, per_bh_state=False):
            if per_bh_state:
                return np.stack([x[key][b, h].double().cpu().numpy() for b, h in group])[:, None]
            return np.stack([x[key][b, :, h].double().cpu().numpy() for b, h in group])[:, :, None]
        h = {k: stack(k) for k in ("wl", "rl", "v", "gamma", "d_o")}
        op = oracle.problem(n, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, U=cfg.U, P=cfg.P,
                            eps=cfg.eps)
        t0 = time.perf_counter()
        oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"])
        oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], None, None, h["d_o"])
        spent += time.perf_counter() - t0
        done += n
        del h
    tokens = done * cfg.T / cfg.H          # a (b, h) slice is 1/H of T tokens' work
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fwd+bwd of {done} of {cfg.B * cfg.H} (b,h) slices of the same workload "
                      f"(T={cfg.T} tokens each, = {tokens:.0f} tokens), {spent:.1f} s on "
                      f"{threads} host threads"}


def decode_step_bytes(cfg, b_io=2):
    """Algorithmic bytes of one autoregressive step over the batch: both
    logit rows, v, gamma and o of every (sequence, head), and the k_w slot
    rows (content and mass) read and written plus the k_r slot rows read."""
    BH = cfg.B * cfg.H
    per = (2 * cfg.S * b_io + 2 * cfg.d_v * b_io + b_io
           + cfg.k_w * 2 * (cfg.d_v + 1) * 4 + cfg.k_r * (cfg.d_v + 1) * 4)
    return BH * per


def bench_decode(args, torch, ram, synth, dev):
    """Autoregressive decoding: args.dec_steps calls of ram_decode_step on the
    state of 256 sequences, inputs from a ring of args.dec_ring pregenerated
    steps (all resident in HBM), replayed from a HIP graph of one ring pass so
    that host launch cost is not timed."""
    cfg = synth.CONFIGS["decode"]
    slot, mass = synth.decode_state(cfg, device=dev, seed=0)
    ring = [synth.decode_step_inputs(cfg, s, device=dev, seed=0) for s in range(args.dec_ring)]
    p = ram.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io, eps=cfg.eps)
    o = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), dtype=cfg.dtype, device=dev)

    def ring_pass():
        for x in ring:
            ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o)

    ring_pass()                                   # warm-up (eager)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ring_pass()
    torch.cuda.synchronize()
    reps = max(1, args.dec_steps // args.dec_ring)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    steps = reps * args.dec_ring
    # per-kernel time: the same ring eagerly with the library's event timing
    ram.ram_prof_enable(True)
    ring_pass()
    torch.cuda.synchronize()
    prof = ram.ram_prof_collect()
    ram.ram_prof_enable(False)
    n, t = prof["decode_step"]
    per_step = decode_step_bytes(cfg)
    achieved = per_step / (t / n * 1e-3) / 1e9
    return {
        "metric": "tokens/sec of autoregressive decode steps on 1 MI355X; achieved HBM GB/s vs peak",
        "value": cfg.B * steps / el, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.dec_ring, "ms_per_step": el * 1e3 / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "RAM-Net autoregressive decode step", "sequences": cfg.B,
                   "H": cfg.H, "S": cfg.S, "k_w": cfg.k_w, "k_r": cfg.k_r, "d_v": cfg.d_v,
                   "io_dtype": "bf16", "state": "f32, 8.6 GB resident",
                   "inputs": f"ring of {args.dec_ring} pregenerated steps",
                   "launch": "HIP graph of one ring pass"},
        "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": per_step},
        "kernels": {k: {"launches": a, "avg_ms": b / a} for k, (a, b) in prof.items()},
    }


def long_bytes(cfg, b_io=2):
    """Algorithmic bytes of the long-context forward: per token-head both
    logit rows, v, gamma and o; per chunk the state (content and mass)
    written, and read back by the next chunk."""
    N = cfg.B * cfg.T * cfg.H
    per_tok = 2 * cfg.S * b_io + 2 * cfg.d_v * b_io + b_io
    nchunk = cfg.T // cfg.chunk
    state = cfg.B * cfg.H * cfg.S * (cfg.d_v + 1) * 4
    return N * per_tok + nchunk * state + (nchunk - 1) * state


def bench_long(args, torch, ram, synth, dev):
    """Long context: a 65,536-token forward as 16 calls of 4,096 tokens, each
    starting from the state the previous one left (chunk inputs pregenerated
    and resident; the first chunk starts from empty slots)."""
    cfg = synth.CONFIGS["long"]
    nchunk = cfg.T // cfg.chunk
    chunks = [synth.chunk_inputs(cfg, c, device=dev, seed=0) for c in range(nchunk)]
    p = ram.problem(cfg.B, cfg.H, cfg.chunk, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io,
                    eps=cfg.eps)
    ws = ram.workspace(p, False, dev)
    o = torch.empty_like(chunks[0]["v"])
    st = [(torch.empty((cfg.B, cfg.H, cfg.S, cfg.d_v), dtype=torch.float32, device=dev),
           torch.empty((cfg.B, cfg.H, cfg.S), dtype=torch.float32, device=dev)) for _ in range(2)]

    def run():
        prev = (None, None)
        for c, x in enumerate(chunks):
            s1, m1 = st[c % 2]
            ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], prev[0], prev[1], o, s1,
                            m1, ws)
            prev = (s1, m1)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / reps
    ram.ram_prof_enable(True)
    run()
    torch.cuda.synchronize()
    prof = ram.ram_prof_collect()
    ram.ram_prof_enable(False)
    n, t = prof["decode_fwd"]
    dec_b = 2 * cfg.B * cfg.chunk * cfg.H * (cfg.S * 2 + 4 + cfg.k_w * 8)
    achieved = dec_b / (t / n * 1e-3) / 1e9
    alg = long_bytes(cfg)
    return {
        "metric": "tokens/sec of a long-context forward (chunked, state carry) on 1 MI355X; "
                  "achieved HBM GB/s vs peak",
        "value": cfg.B * cfg.T / el, "unit": "tokens/s", "n_gpus": 1, "steps": reps,
        "warmup": max(1, args.warmup), "ms_per_step": el * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "RAM-Net forward, 65,536 tokens in 16 chunks of 4,096",
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "chunk": cfg.chunk, "S": cfg.S,
                   "k_w": cfg.k_w, "k_r": cfg.k_r, "d_v": cfg.d_v, "io_dtype": "bf16",
                   "state": "f32, carried between chunks"},
        "roofline": {"bound": "hbm", "kernel": "decode_fwd", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": dec_b},
        "step_hbm": {"algorithmic_bytes": alg, "achieved_GBps": alg / el / 1e9,
                     "frac_of_peak": alg / el / 1e9 / PEAK_HBM_GBS},
        "kernels": {k: {"launches": a, "avg_ms": b / a} for k, (a, b) in prof.items()},
    }


def bench_stream(args, torch, ram, dev):
    """HBM streaming roofs with the decoders' access pattern (ram_stream_probe):
    read-only and copy (read a row, write a row) of a 4 GiB buffer, per probe
    variant, median of args.steps repetitions after args.warmup; torch's own
    copy of the same buffer for reference.  GB/s count the bytes read plus the
    bytes written."""
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(7)
    reps = max(3, args.steps)

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b) * 1e-3)
        return sorted(out)[len(out) // 2]

    read, copy = {}, {}
    for v, name in enumerate(ram.STREAM_PROBE_VARIANTS):
        read[name] = n / timed(lambda: ram.ram_stream_probe(0, v, src, dst)) / 1e9
        copy[name] = 2 * n / timed(lambda: ram.ram_stream_probe(1, v, src, dst)) / 1e9
    torch_copy = 2 * n / timed(lambda: dst.copy_(src)) / 1e9
    own = ram.STREAM_PROBE_VARIANTS[5]   # the decode backward's pattern
    return {
        "metric": "HBM streaming roofs of the decoders' access pattern on 1 MI355X",
        "value": copy[own], "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None, "data": "synthetic",
        "config": {"workload": "stream 4 GiB: read-only and copy", "bytes": n,
                   "value_is": f"copy, {own}"},
        "read_GBps": read, "copy_GBps": copy, "torch_copy_GBps": torch_copy,
        "read_frac_of_peak": {k: v / PEAK_HBM_GBS for k, v in read.items()},
        "copy_frac_of_peak": {k: v / PEAK_HBM_GBS for k, v in copy.items()},
    }


def copy_calibration(steps=5):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--config", default="1.3b",
                    help="workload: 1.3b (default, the measured one), 340m, 1.3b-uniform "
                         "(no hot-slot bias) or 1.3b-u2 (U = 2 digits of 64): fwd+bwd "
                         "steps; decode: autoregressive steps of 256 sequences; long: "
                         "a 65,536-token forward in 4,096-token chunks with state carry; "
                         "stream: the HBM read and copy roofs of the decoders' pattern")
    ap.add_argument("--flush", action="store_true",
                    help="fwd+bwd configs: overwrite a 1 GiB buffer before every step (evicts "
                         "L2 and the 256 MB Infinity Cache) and time only the steps")
    ap.add_argument("--gated", action="store_true",
                    help="fwd+bwd configs: the gated read-out y = sigmoid(gate) * RMSNorm(o) "
                         "fused into the read (ram_forward_gated / ram_backward_gated)")
    ap.add_argument("--dec-steps", type=int, default=1024,
                    help="decode: autoregressive steps per timed run")
    ap.add_argument("--dec-ring", type=int, default=64,
                    help="decode: distinct pregenerated step inputs, cycled")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the core shards over (batch, head) "
                                   "with no communication between the shards, so N GPUs run N "
                                   "independent copies of the one-GPU workload", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import linear_attention_ram_amd as ram
    from linear_attention_ram_amd import synth

    dev = torch.device("cuda:0")
    if args.config == "decode":
        print(json.dumps(bench_decode(args, torch, ram, synth, dev)))
        return
    if args.config == "long":
        print(json.dumps(bench_long(args, torch, ram, synth, dev)))
        return
    if args.config == "stream":
        print(json.dumps(bench_stream(args, torch, ram, dev)))
        return
    if args.config == "1.3b-uniform":
        cfg = synth.CONFIGS["1.3b"].with_(zipf=None, name="1.3b-uniform")
    else:
        cfg = synth.CONFIGS[args.config]
    x = synth.layer_inputs(cfg, device=dev, seed=0)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io, eps=cfg.eps,
                    U=cfg.U, P=cfg.P)
    ws = ram.workspace(p, True, dev)
    o = torch.empty_like(x["v"])
    slot1 = torch.empty((cfg.B, cfg.H, cfg.S, cfg.d_v), dtype=torch.float32, device=dev)
    mass1 = torch.empty((cfg.B, cfg.H, cfg.S), dtype=torch.float32, device=dev)
    d_wl, d_rl = torch.empty_like(x["wl"]), torch.empty_like(x["rl"])
    d_v, d_g = torch.empty_like(x["v"]), torch.empty_like(x["gamma"])
    if args.gated:
        gx = synth.gate_inputs(cfg, device=dev, seed=0)
        ep = ram.epilogue(p, gx["gate"], gx["gain"], 1e-6)
        d_gate = torch.empty_like(gx["gate"])
        d_gain = torch.empty_like(gx["gain"])

    def step():
        if args.gated:
            ram.ram_forward_gated(p, ep, x["wl"], x["rl"], x["v"], x["gamma"], None, None, o,
                                  slot1, mass1, ws)
            ram.ram_backward_gated(p, ep, ws, x["wl"], x["rl"], x["v"], x["gamma"], None, None,
                                   gx["d_y"], None, None, d_wl, d_rl, d_v, d_g, d_gate, d_gain)
            return
        ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], None, None, o, slot1, mass1, ws)
        ram.ram_backward(p, ws, x["wl"], x["rl"], x["v"], x["gamma"], None, None, x["d_o"],
                         None, None, d_wl, d_rl, d_v, d_g)

    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.flush else None

    def flush(i):
        if flush_buf is not None:
            flush_buf.fill_(i & 255)

    for i in range(args.warmup):
        flush(i)
        step()
    torch.cuda.synchronize()
    if args.flush:
        # each step bracketed by events on the current stream (the library
        # joins its own stream back into it), the flush left out
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (a, b) in enumerate(evs):
            flush(i)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        elapsed = sum(a.elapsed_time(b) for a, b in evs) * 1e-3
    else:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    # second pass: per-kernel events
    ram.ram_prof_enable(True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush(i)
        step()
    torch.cuda.synchronize()
    prof = ram.ram_prof_collect()
    ram.ram_prof_enable(False)

    ms_step = elapsed * 1e3 / args.steps
    tokens = cfg.B * cfg.T
    fwd_b, bwd_b = algorithmic_bytes(cfg)
    kernels = {k: {"launches": n, "avg_ms": t / n} for k, (n, t) in sorted(prof.items())}
    n_bwd, t_bwd = prof["decode_bwd"]
    dom_bytes = decode_bwd_bytes(cfg)
    achieved = dom_bytes / (t_bwd / n_bwd * 1e-3) / 1e9
    traffic = measured_traffic() if cfg.name == "1.3b" else None
    step_gbs = (fwd_b + bwd_b) / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"RAM-Net attention core, {cfg.name}-layer shape, fwd+bwd",
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "S": cfg.S, "k_w": cfg.k_w,
                   "k_r": cfg.k_r, "d_v": cfg.d_v, "U": cfg.U, "P": cfg.P,
                   "io_dtype": "bf16", "state": "f32",
                   "address_bias": f"Zipf({cfg.zipf}) per slot" if cfg.zipf else "none",
                   "tokens_per_step": tokens,
                   "caches": ("flushed before every step (1 GiB overwrite)" if args.flush
                              else "warm (no flush between steps)"),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "decode_bwd", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes},
        "step_hbm": {"algorithmic_bytes": fwd_b + bwd_b, "achieved_GBps": step_gbs,
                     "frac_of_peak": step_gbs / PEAK_HBM_GBS, "target_frac": 0.60,
                     "meets_target": step_gbs / PEAK_HBM_GBS >= 0.60},
        "kernels": kernels,
    }
    if args.gated:
        # kernel bytes of the fused read epilogue: the k_r read contributions
        # (io) of every row and the gate read, y written; backward: the same
        # contributions, gate and d_y read, d_o and d_gate written
        N, b_io = cfg.B * cfg.T * cfg.H, 2
        epi_b = {"epilogue_fwd": N * cfg.d_v * b_io * (cfg.k_r + 2),
                 "epilogue_bwd": N * cfg.d_v * b_io * (cfg.k_r + 4)}
        out["config"]["read_out"] = "gated: sigmoid(gate) * RMSNorm(o), fused"
        out["epilogue_roofline"] = {
            k: {"bytes": b, "GBps": b / (prof[k][1] / prof[k][0] * 1e-3) / 1e9,
                "frac": b / (prof[k][1] / prof[k][0] * 1e-3) / 1e9 / PEAK_HBM_GBS}
            for k, b in epi_b.items()}
    if not args.no_cpu_baseline and not args.gated:
        # every core the process may run on, unless the box's share of the
        # host (OMP_NUM_THREADS) is smaller
        affinity = len(os.sched_getaffinity(0))
        threads = affinity
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():
            threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
        out["cpu_baseline"] = cpu_baseline(cfg, x, threads, args.cpu_budget)
        out["cpu_baseline"]["affinity_cores"] = affinity
    print(json.dumps(out))


if __name__ == "__main__":
    main()
