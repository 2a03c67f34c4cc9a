#!/usr/bin/env python3
"""Throughput of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bulk|prefill]
                    [--no-parts] [--no-cpu] [--no-variants]

A step is one ssm_scan_fwd call (dt, scan, readout, skip, gate, final state;
conv1d + SiLU and the conv cache too for the prefill) over one batch of the
workload, with every input already resident in HBM.  The default workload is
the bandwidth-bound bulk scan (batch 8, L 4096, E 7680, N 16, bf16 u/dt/z/B/C,
bf16 y), on which the HBM bar is judged; --workload prefill times the Bit-Axon
layer prefill (batch 1, L 2048, E 7680, conv1d k=4, rank-1 dt).  Inputs are
the seeded synthetic recipes of ssm_workloads.py.

Prints ONE JSON line.  Besides the throughput it carries
* roofline: the main scan kernel's duration, measured with HIP events that the
  library records on its own launch stream around that kernel, against the
  HBM roofline (the workload's algorithmic bytes over that duration), plus the
  same for the whole call (every kernel of the step, back-to-back launches);
* variants: the same workload with A as a model stores it (fp32 -exp(log n))
  and on the general path (random per-channel A, dt off the clip), which take
  the kernel's slower decay forms;
* cpu_baseline: the float64 oracle on the same workload on this host's CPU
  cores (channels sharded over worker processes), plus one core on one shard;
* parts: the other entry points at their workloads (prefill or bulk scan,
  8-layer decode step, chunked SSD, SSD-form decode step, backward, the whole
  layer forward with its two projection GEMMs), each with its own roofline.
Counters of HBM traffic come from rocprofv3 runs recorded in profiles/; each
is reported only while its kernel's sources still hash to the recorded value.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan tokens/s and achieved HBM GB/s (% of peak) at E=7680, N=16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix, published

# Algorithmic work per unit, counted from the definition of each step (each
# input read once, each output written once; FMA = 2 flops, exp/log/div = 1).
# Scan flops per channel-step: decay 16 x (mul + exp) = 32; state 1 + 16 x (mul
# + fma) = 49; readout 16 fma + D fma = 34; gate SiLU + mul = 5: 120.  The conv
# (4 fma = 8), SiLU of its output (4) and the rank-1 dt with softplus and clip
# (6) add 18 for the layer prefill.
FLOPS_PER_CH_STEP = {"prefill": 138.0, "bulk": 120.0}
# The backward's main walk per channel-step (bwd_main): the forward recomputed
# over the segment (decay 16 x (mul + exp) = 32, update 1 + 16 x 2 = 33,
# dt and u 6), then the reverse step: the state gradient G = dyc C + a G'
# (16 x 3 = 48), dA and dt terms (16 x 2 + 16 x 2 = 64), du (16 x 2 + 2 = 34),
# dB and dC (16 x 2 = 32, their channel sums not counted), dz and the SiLU
# derivatives (8): 257.
BWD_FLOPS_PER_CH_STEP = 257.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=("prefill", "bulk"), default="bulk")
    ap.add_argument("--no-variants", action="store_true", help="skip the model-A and general-path timings")
    ap.add_argument("--split", type=int, default=0,
                    help="time segments per sequence for the scan (0: the library's choice)")
    ap.add_argument("--no-parts", action="store_true", help="skip the decode / SSD / other-scan lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only", choices=("prefill", "bulk", "bulk_general", "prefill_general", "decode", "ssd",
                                       "ssd_decode", "layer", "in_proj", "out_proj", "scan_bwd", "copy"),
                    default=None,
                    help="run just this workload's timed loop, no JSON line (for profiler runs); 'copy' "
                         "copies 1 GiB device to device, the calibration for the HBM byte counters")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------- helpers

# The HIP sources each recorded counter profile depends on (its kernel's own
# files and the shared device header); a profile is used only while they hash
# to the recorded value.
SCAN_SOURCES = ("scan_fused.hip", "scan_fused_impl.h", "scan_xy_bb.hip", "scan_xy_bf.hip", "scan_xy_fb.hip",
                "scan_xy_ff.hip")
# the kernels of one ssm_scan_fwd call, in launch order: the time-split
# kernels (the summary pass and composition run only when the sequence is
# cut), or the blocked single pass (its table packing, then the scan)
SCAN_CALL_KERNELS = ("pack", "pass1", "compose", "main")
BLOCKED_CALL_KERNELS = ("blkpack", "blkmain")
KERNEL_SOURCES = {
    **{f"scan_{k}_{w}": SCAN_SOURCES for k in SCAN_CALL_KERNELS for w in ("prefill", "bulk")},
    **{f"scan_{k}_bulk": ("scan_blocked.hip",) for k in BLOCKED_CALL_KERNELS},
    "decode": ("decode_step.hip",), "ssd": ("ssd_chunk.hip",), "ssd_decode": ("ssd_decode.hip",),
    "gemm_in_proj": ("gemm.hip",), "gemm_out_proj": ("gemm.hip",), "scan_bwd": ("scan_bwd.hip",),
}


def sources_digest(kernel_key):
    """sha256 over the HIP sources of one kernel (plus the shared device header)."""
    d = os.path.join(ROOT, "selective_state_space_03_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kernel_key] + ("ssm_device.h",)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_key):
    """HBM bytes per launch from profiles/pmc_traffic.txt (FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by the copy-kernel calibration), or
    None when none is recorded for the kernel's current sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get(f"{kernel_key}.sources") != sources_digest(kernel_key):
        return None
    try:
        fetch = float(rec[f"{kernel_key}.fetch_kib"]) * float(rec["copy.fetch_factor"])
        write = float(rec[f"{kernel_key}.write_kib"]) * float(rec["copy.write_factor"])
    except KeyError:
        return None
    return (fetch + write) * 1024.0


def blocked_path(which, split):
    """Whether the library runs the blocked single pass for this workload: the
    bulk recipe (bf16 u / z / E-wide dt, no conv, 960 channel groups) with the
    library's own choice (time_split 0) or asked for (time_split -1)."""
    return which == "bulk" and split in (0, -1)


def main_kernel_key(which, split):
    return "scan_blkmain_bulk" if blocked_path(which, split) else f"scan_main_{which}"


def call_traffic(workload, split=0):
    """HBM bytes of every kernel of one scan call (recorded profiles), summed;
    None unless each kernel the call ran has a current record."""
    blocked = blocked_path(workload, split)
    total, seen = 0.0, 0
    for k in (BLOCKED_CALL_KERNELS if blocked else SCAN_CALL_KERNELS):
        t = recorded_traffic(f"scan_{k}_{workload}")
        if t is None:
            continue
        total += t
        seen += 1
    main = recorded_traffic(main_kernel_key(workload, split))
    return total if (seen and main is not None) else None


def dev_tensor(torch, w, key, device):
    a = w.arrays.get(key)
    if a is None:
        return None
    if key in w.bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class KernelTimer:
    """Per-launch HIP events that the library records around its main kernel."""

    def __init__(self, torch, ssm, n):
        self.torch, self.ssm = torch, ssm
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]
        self.i = 0

    def arm(self):
        s, e = self.pairs[self.i]
        self.ssm.set_timing_events(s, e)
        self.i += 1

    def disarm(self):
        self.ssm.set_timing_events(None, None)

    def mean_ms(self):
        ts = [s.elapsed_time(e) for s, e in self.pairs[: self.i]]
        return float(np.mean(ts)), float(np.median(ts))


def timed_loop(torch, ssm, calls, steps, warmup, per_step=1, per_launch=True):
    """Warm up, then run `steps` steps (each `per_step` consecutive calls from the
    rotating list) between two synchronisations.  Returns wall ms per step and
    the main kernel's mean and median duration per call: from the HIP events
    the library records around that kernel (per_launch), or, for entry points
    that launch nothing else, from two events around the whole timed region
    divided by the number of calls (back-to-back launches, gaps included)."""
    n = len(calls)
    for i in range(warmup * per_step):
        calls[i % n].run()
    torch.cuda.synchronize()
    timer = KernelTimer(torch, ssm, steps * per_step) if per_launch else None
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for i in range(steps * per_step):
        if timer:
            timer.arm()
        calls[i % n].run()
    r1.record()
    if timer:
        timer.disarm()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    if timer:
        kmean, kmed = timer.mean_ms()
    else:
        kmean = kmed = r0.elapsed_time(r1) / (steps * per_step)
    return wall_ms, kmean, kmed


# ------------------------------------------------------------------- workloads

def make_scan_workload(W, which, variant="base"):
    """The headline recipes (variant "base"), A as a model stores it
    ("log_init": fp32 -exp(fp32 log(1..16)), which breaks the exact power
    structure), or the general path ("general": random per-channel A and the
    dt recipe shifted off the clip)."""
    kw = {"base": {}, "log_init": dict(a_init="log_init"),
          "general": dict(a_init="random", unsaturated=True)}[variant]
    return W.scan_prefill(**kw) if which == "prefill" else W.scan_bulk(**kw)


def scan_calls(torch, ssm, W, which, sets, device, stream=None, split=0, w=None):
    w = w if w is not None else make_scan_workload(W, which)
    o, d = w.opts, w.dims
    calls = []
    for _ in range(sets):
        x, A, B, C, dt = (dev_tensor(torch, w, k, device) for k in ("x", "A", "B", "C", "dt"))
        y = torch.empty((d["batch"], d["seqlen"], d["dim"]), dtype=torch.bfloat16, device=device)
        st = torch.empty((d["batch"], d["dim"], d["d_state"]), dtype=torch.float32, device=device)
        cc = torch.empty((d["batch"], d["dim"], 3), dtype=torch.float32, device=device) if o["conv"] else None
        calls.append(ssm.scan_fwd(
            x, A, B, C, dt, D=dev_tensor(torch, w, "D", device), z=dev_tensor(torch, w, "z", device),
            conv_w=dev_tensor(torch, w, "conv_w", device) if o["conv"] else None, conv_cache_out=cc,
            dt_rank1=o["dt_rank1"], dt_w=dev_tensor(torch, w, "dt_w", device),
            dt_bias=dev_tensor(torch, w, "dt_bias", device), dt_softplus=o["dt_softplus"],
            dt_min=o["dt_min"], dt_max=o["dt_max"], ssm_state_out=st, y=y, stream=stream, time_split=split, prepare=True))
    Bt, L, E, N = d["batch"], d["seqlen"], d["dim"], d["d_state"]
    # algorithmic bytes: x/u, z (and E-wide dt) in, y out (bf16); B, C (bf16)
    # and the rank-1 r; per-channel parameters; state (and conv cache) out.
    ew = 2 * Bt * L * E * (3 if which == "prefill" else 4)
    small = 2 * 2 * Bt * L * N + (4 * Bt * L if which == "prefill" else 0)
    params = 4 * E * (N + 1 + (2 + 4 if which == "prefill" else 1))
    outs = 4 * Bt * E * N + (4 * Bt * E * 3 if o["conv"] else 0)
    return w, calls, dict(batch=Bt, seq_len=L, dim=E, d_state=N, bytes=ew + small + params + outs)


def decode_calls(torch, ssm, W, layers, ring, device, stream=None):
    """Config of the batched decode step: batch 64, E 7680, N 16, fp32; `layers`
    independent state/cache sets (like stacked layers, 37 MB each) so the
    states stream from HBM instead of the last-level cache."""
    w = W.decode_stream(prefill=0, steps=ring)
    t = lambda k: torch.from_numpy(np.ascontiguousarray(w.arrays[k])).to(device)
    X, Z, R, Bm, Cm = (t(k) for k in ("x", "z", "dt", "B", "C"))
    A, D, cw, dw, db = (t(k) for k in ("A", "D", "conv_w", "dt_w", "dt_bias"))
    g = torch.Generator(device="cpu").manual_seed(44)
    Bt, E, N = w.dims["batch"], w.dims["dim"], w.dims["d_state"]
    states = [torch.randn((Bt, E, N), generator=g).mul_(0.1).to(device) for _ in range(layers)]
    caches = [torch.randn((Bt, E, 3), generator=g).to(device) for _ in range(layers)]
    ys = [torch.empty((Bt, E), dtype=torch.float32, device=device) for _ in range(layers)]
    calls = []
    for s in range(ring):
        for l in range(layers):
            calls.append(ssm.decode_step(X[s], A, Bm[s], Cm[s], R[s], states[l], conv_cache=caches[l], D=D,
                                         z=Z[s], conv_w=cw, dt_rank1=True, dt_w=dw, dt_bias=db,
                                         dt_min=w.opts["dt_min"], dt_max=w.opts["dt_max"], y=ys[l],
                                         stream=stream, prepare=True))
    # per call: state r+w, cache r+w, x, z, y (fp32), r, B, C, parameters
    byts = 2 * 4 * Bt * E * N + 2 * 4 * Bt * E * 3 + 3 * 4 * Bt * E + 4 * Bt * (1 + 2 * N) + 4 * E * (N + 4 + 3)
    return calls, dict(batch=Bt, dim=E, d_state=N, layers=layers, bytes=byts)


def ssd_decode_calls(torch, ssm, W, layers, ring, device, stream=None):
    """Decode step of the multi-head scan at serving size: batch 64, 80 heads x
    96, 1 group, N 64, bf16 x/B/C/out, fp32 state (126 MB per state set);
    `layers` state sets so the states stream from HBM."""
    w = W.ssd_decode(steps=ring)
    d = w.dims
    X, R, Bm, Cm = (dev_tensor(torch, w, k, device) for k in ("x", "dt", "B", "C"))
    A, D, db = (dev_tensor(torch, w, k, device) for k in ("A", "D", "dt_bias"))
    Bt, H, P, G, N = (d[k] for k in ("batch", "nheads", "headdim", "ngroups", "d_state"))
    g = torch.Generator(device="cpu").manual_seed(45)
    states = [torch.randn((Bt, H, P, N), generator=g).to(device) for _ in range(layers)]
    outs = [torch.empty((Bt, H, P), dtype=torch.bfloat16, device=device) for _ in range(layers)]
    xs = [X[:, s].contiguous() for s in range(ring)]
    rs = [R[:, s].contiguous() for s in range(ring)]
    bs = [Bm[:, s].contiguous() for s in range(ring)]
    cs = [Cm[:, s].contiguous() for s in range(ring)]
    calls = []
    for s in range(ring):
        for l in range(layers):
            calls.append(ssm.chunk_decode_step(xs[s], rs[s], A, bs[s], cs[s], states[l], D=D, dt_bias=db,
                                               dt_min=w.opts["dt_min"], dt_max=w.opts["dt_max"], out=outs[l],
                                               stream=stream, prepare=True))
    # per call: state r+w (fp32), x and out (bf16), dt (fp32), B and C (bf16), A/D/bias
    byts = 2 * 4 * Bt * H * P * N + 2 * 2 * Bt * H * P + 4 * Bt * H + 2 * 2 * Bt * G * N + 4 * 3 * H
    return calls, dict(batch=Bt, nheads=H, headdim=P, ngroups=G, d_state=N, layers=layers, bytes=byts)


def decode_graph(torch, ssm, W, device, layers=8, ring=16, make=None):
    """The decode steps of `ring` tokens through `layers` state sets, captured
    once in a HIP graph (as a serving loop would run them): replays time the
    kernels without the Python launch cost."""
    stream = torch.cuda.Stream(device)
    calls, cfg = (make or decode_calls)(torch, ssm, W, layers, ring, device, stream=stream)
    stream.wait_stream(torch.cuda.current_stream(device))
    for c in calls:  # warm-up outside the graph
        c.run()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c.run()
    torch.cuda.synchronize()
    return graph, len(calls), cfg


def capture_each(torch, calls, stream):
    """One HIP graph per prepared call (all on `stream`), captured after a
    warm-up run of each call."""
    stream.wait_stream(torch.cuda.current_stream())
    for c in calls:
        c.run()
    stream.synchronize()
    graphs = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            c.run()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_all(torch, calls, stream):
    """One HIP graph holding one step on each buffer set, in order (calls
    already warmed up by capture_each)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c.run()
    torch.cuda.synchronize()
    return g


def timed_graphs(torch, graphs, whole, steps, warmup):
    """Warm up, then run exactly `steps` steps between two synchronisations:
    replays of `whole` (one step per buffer set) and, for the remainder, of
    the single-step graphs.  Returns wall ms per step."""
    n = len(graphs)
    for i in range(warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // n):
        whole.replay()
    for i in range(steps % n):
        graphs[i].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def graph_time(torch, graph, launches, replays):
    """Mean ms per launch over `replays` graph replays (events around them)."""
    graph.replay()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(replays):
        graph.replay()
    r1.record()
    torch.cuda.synchronize()
    return r0.elapsed_time(r1) / (replays * launches)


def ssd_calls(torch, ssm, W, device):
    w = W.ssd_long()
    d = w.dims
    x, dtr, A, B, C, D, db = (dev_tensor(torch, w, k, device) for k in ("x", "dt", "A", "B", "C", "D", "dt_bias"))
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=device)
    st = torch.empty((d["batch"], d["nheads"], d["headdim"], d["d_state"]), dtype=torch.float32, device=device)
    call = ssm.chunk_scan_fwd(x, dtr, A, B, C, chunk_size=d["chunk_size"], D=D, dt_bias=db,
                              dt_softplus=w.opts["dt_softplus"], dt_min=w.opts["dt_min"], dt_max=w.opts["dt_max"],
                              state_out=st, out=out, prepare=True)
    Bt, L, H, P, G, N, Q = (d[k] for k in ("batch", "seqlen", "nheads", "headdim", "ngroups", "d_state",
                                            "chunk_size"))
    byts = 2 * 2 * Bt * L * H * P + 2 * 2 * Bt * L * G * N + 4 * Bt * L * H + 4 * Bt * H * P * N + 4 * 3 * H
    # dense flops: C.B^T per chunk and group, intra-chunk (causal half), state
    # readout and chunk-state update per head
    nch = L // Q
    flops = Bt * nch * (2 * Q * Q * N * G + H * (Q * Q * P + 2 * Q * N * P + 2 * Q * N * P))
    return [call], dict(batch=Bt, seq_len=L, nheads=H, headdim=P, d_state=N, chunk_size=Q, bytes=byts,
                        flops=flops)


def layer_calls(torch, ssm, W, device):
    """The whole Axon-SSM layer forward at the page's sizes (batch 1, 2048
    tokens, D 2560, E 7680, N 16), random bf16 weights, bf16 output."""
    w = W.layer_prefill()
    o, d = w.opts, w.dims
    args = [dev_tensor(torch, w, k, device) for k in ("hidden", "W_in", "conv_w", "W_x", "dt_w", "A", "W_out")]
    T, Dm, E, N = d["batch"] * d["seqlen"], d["d_model"], d["dim"], d["d_state"]
    out = torch.empty((d["batch"], d["seqlen"], Dm), dtype=torch.bfloat16, device=device)
    call = ssm.layer_fwd(*args, dt_bias=dev_tensor(torch, w, "dt_bias", device), D=dev_tensor(torch, w, "D", device),
                         dt_min=o["dt_min"], dt_max=o["dt_max"], out=out, prepare=True)
    # dense flops of the projections plus the scan's per channel-step work
    flops = 2 * T * Dm * 2 * E + 2 * T * E * (2 * N + 1) + 2 * T * E * Dm + FLOPS_PER_CH_STEP["prefill"] * T * E
    return [call], dict(batch=d["batch"], seq_len=d["seqlen"], d_model=Dm, dim=E, d_state=N, flops=flops)


def bwd_calls(torch, ssm, W, device):
    """Backward of the layer-prefill scan (batch 1, 2048 tokens, E 7680, N 16):
    all gradients, upstream gradient dy ~ N(0,1) fp32."""
    w = W.scan_prefill()
    o, d = w.opts, w.dims
    t = lambda k: dev_tensor(torch, w, k, device)  # noqa: E731
    g = torch.Generator(device="cpu").manual_seed(47)
    dy = torch.randn((d["batch"], d["seqlen"], d["dim"]), generator=g).to(device)
    call = ssm.scan_bwd(t("x"), t("A"), t("B"), t("C"), t("dt"), dy, D=t("D"), z=t("z"), conv_w=t("conv_w"),
                        dt_rank1=True, dt_w=t("dt_w"), dt_bias=t("dt_bias"), dt_min=o["dt_min"], dt_max=o["dt_max"],
                        prepare=True)
    Bt, L, E, N = d["batch"], d["seqlen"], d["dim"], d["d_state"]
    # algorithmic bytes: inputs x, z (bf16), dy (fp32), r, B, C once; gradients dx, dz (fp32), dB, dC, dr
    byts = Bt * L * E * (2 + 2 + 4 + 4 + 4) + Bt * L * (4 + 4 + 2 * N * 2 + 2 * N * 4)
    return [call], dict(batch=Bt, seq_len=L, dim=E, d_state=N, bytes=byts)


GEMM_SHAPES = {"in_proj": (2048, 2560, 15360, "bf16"), "out_proj": (2048, 7680, 2560, "f32")}


def gemm_calls(torch, ssm, which, device):
    """One layer projection through ssm_linear_fwd at the layer prefill's shape:
    in_proj (2048 x 2560 -> 15360, bf16 input) or out_proj (2048 x 7680 -> 2560,
    fp32 input entering as a bf16 value/remainder pair)."""
    M, K, N, xdt = GEMM_SHAPES[which]
    g = torch.Generator(device="cpu").manual_seed(46)
    x = torch.randn((M, K), generator=g).to(device, torch.bfloat16 if xdt == "bf16" else torch.float32)
    wt = (torch.randn((N, K), generator=g) / K ** 0.5).to(device, torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.float32, device=device)
    call = ssm.linear_fwd(x, wt, out=out, prepare=True)
    # MFMA work: a value/remainder pair doubles the products of an fp32 input
    return [call], dict(M=M, K=K, N=N, x_dtype=xdt, flops=2 * M * N * K,
                        mfma_flops=2 * M * N * K * (2 if xdt == "f32" else 1))


COPY_GBS = None  # read + write rate of a plain 1 GiB device-to-device copy, measured once per run


def copy_rate(torch, device):
    """GB/s (read + write) of torch's device-to-device copy of 1 GiB: the
    practical streaming ceiling of this machine, beside the published 8 TB/s."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(5):
        dst.copy_(src)
    r1.record()
    torch.cuda.synchronize()
    ms = r0.elapsed_time(r1) / 5
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def roof_hbm(nbytes, kernel_ms, traffic):
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    if COPY_GBS:
        out["frac_of_copy"] = round(gbs / COPY_GBS, 4)
    return out


# ----------------------------------------------------------------------- CPU

_CPU = {}


def _slice64(w, key, ch, axis):
    """Channels `ch` of a workload array along `axis`, widened to float64 (the
    bf16 bit patterns are sliced before they are widened)."""
    a = np.take(w.arrays[key], ch, axis=axis)
    if key in w.bf16:
        return W_bf16_to_f64(a)
    return np.asarray(a, np.float64)


def W_bf16_to_f64(bits):
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _oracle_shard(ch):
    """The float64 oracle on channels `ch` of the workload in _CPU, on one core
    (BLAS limited to one thread).  Returns the seconds it took."""
    from oracle import ssm_oracle as O
    from threadpoolctl import threadpool_limits
    w = _CPU["w"]
    o = w.opts
    ch = np.asarray(ch)
    kw = dict(D=_slice64(w, "D", ch, 0), z=_slice64(w, "z", ch, 2), dt_bias=_slice64(w, "dt_bias", ch, 0),
              dt_softplus=o["dt_softplus"], dt_min=float(o["dt_min"]), dt_max=float(o["dt_max"]))
    if o["conv"]:
        kw["conv_w"] = _slice64(w, "conv_w", ch, 0)
    if o["dt_rank1"]:
        kw["dt_raw"] = w.f64("dt")
        kw["dt_w"] = _slice64(w, "dt_w", ch, 0)
    else:
        kw["dt"] = _slice64(w, "dt", ch, 2)
    x, A = _slice64(w, "x", ch, 2), _slice64(w, "A", ch, 0)
    B, C = w.f64("B"), w.f64("C")
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.ssm_layer_scan(x, A, B, C, **kw)
        return time.perf_counter() - t0


def cpu_baseline(w, name):
    """The float64 oracle on the whole workload on this host: the channels
    (independent given B, C and dt) split into one shard per available core,
    each run by its own process; then one core on one shard, scaled to all
    channels.  Runs before anything touches the GPU (the workers are forked)."""
    import multiprocessing
    cores = len(os.sched_getaffinity(0))
    E = w.dims["dim"]
    shards = np.array_split(np.arange(E), cores)
    _CPU["w"] = w
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        per = pool.map(_oracle_shard, shards)
    wall = time.perf_counter() - t0
    one = _oracle_shard(shards[0])
    _CPU.clear()
    tokens = w.dims["batch"] * w.dims["seqlen"]
    one_all = one * E / len(shards[0])
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(tokens / wall, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {name} workload ({w.dims['batch']} x {w.dims['seqlen']} tokens x {E} channels), "
                      f"float64 numpy, its channels split into {cores} shards run by {cores} processes "
                      f"({wall:.1f} s wall, slowest shard {max(per):.1f} s; one thread each)",
            "single_core": {"value": round(tokens / one_all, 1), "unit": "tokens/s", "cores": 1,
                            "sample": f"one shard of {len(shards[0])} channels on one core ({one:.1f} s), "
                                      f"scaled to {E} channels"},
            "cpu_model": cpu}


# ---------------------------------------------------------------------- main

WORKLOAD_NAMES = {"bulk": "Bandwidth-bound bulk scan", "prefill": "Bit-Axon SSM layer prefill"}
VARIANT_NOTES = {
    "log_init": "A = -exp(log(1..16)) rounded to fp32 as a model stores it (5 of the 16 entries an ulp or two off "
                "-(n+1), so the decays are one exponential each); dt recipe unchanged",
    "general": "A = -exp(U[0, ln 16]) drawn per (channel, state); dt recipe shifted off the clip (bias N(-4, 1)): "
               "one exponential per state and step, softplus on every step",
}


def scan_step_timing(torch, ssm, calls, steps, warmup, stream):
    """Times the steps three ways: launched back to back with the library's HIP
    events around each call's main kernel (the kernel roofline's source),
    replayed from a HIP graph, and launched back to back with two events
    around the whole region (the whole call).  Returns a dict of ms."""
    with torch.cuda.stream(stream):
        eager, kmean, kmed = timed_loop(torch, ssm, calls, steps, warmup)
    graphs = capture_each(torch, calls, stream)
    whole = capture_all(torch, calls, stream)
    graph_ms = timed_graphs(torch, graphs, whole, steps, warmup)
    del graphs, whole
    with torch.cuda.stream(stream):
        launch_ms, call_ms, _ = timed_loop(torch, ssm, calls, steps, warmup, per_launch=False)
    return dict(eager=eager, kmean=kmean, kmed=kmed, graph=graph_ms, launch=launch_ms, call=call_ms,
                step=min(graph_ms, launch_ms))


def scan_line(which, cfg, t, tokens, split=0):
    """Throughput and rooflines of one scan workload from its timings."""
    byts = cfg["bytes"]
    ch_steps = tokens * cfg["dim"]
    gflop = FLOPS_PER_CH_STEP[which] * ch_steps / 1e9
    kgbs = byts / (t["kmean"] * 1e-3) / 1e9
    cgbs = byts / (t["call"] * 1e-3) / 1e9
    blocked = blocked_path(which, split)
    traffic = recorded_traffic(main_kernel_key(which, split))
    roof = {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": ("scan_blk_kernel (the whole sequence in one pass of 16-step blocks)" if blocked
                       else "scan_kernel (full pass)"),
            "kernel_us": round(t["kmean"] * 1e3, 2),
            "algorithmic_bytes": byts,
            "whole_call": {"us": round(t["call"] * 1e3, 2), "achieved": round(cgbs, 1),
                           "frac": round(cgbs / HBM_PEAK_GBS, 4), "traffic": call_traffic(which, split),
                           "note": ("every kernel of one call (the per-block table packing and the scan)" if blocked
                                    else "every kernel of one call (B/C packing, and with a time split the "
                                         "summary pass and composition)") +
                                   ", back-to-back launches; traffic summed over them"},
            "alu": {"achieved_tflops": round(gflop / t["kmean"], 2), "peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                    "frac": round(gflop / t["kmean"] / FP32_VECTOR_PEAK_TFLOPS, 4),
                    "frac_of_unpacked": round(gflop / t["kmean"] / (FP32_VECTOR_PEAK_TFLOPS / 2), 4),
                    "flops_per_channel_step": FLOPS_PER_CH_STEP[which]}}
    if COPY_GBS:
        roof["frac_of_copy"] = round(kgbs / COPY_GBS, 4)
        roof["whole_call"]["frac_of_copy"] = round(cgbs / COPY_GBS, 4)
    return roof


def seqlen_sweep(torch, ssm, W, device, lengths=(512, 2048, 8192, 32768)):
    """The layer-prefill recipe (batch 1, E 7680) at several sequence lengths:
    time per call, tokens/s, the device memory the call needs beyond its
    inputs and outputs (the library's workspace: packed B/C rows and segment
    summaries), the peak of device memory allocated for the call's tensors
    while it runs (measured: inputs, outputs and workspace), beside what
    storing every state (L, E, N) in fp32 would take."""
    rows = []
    for L in lengths:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated(device)
        torch.cuda.reset_peak_memory_stats(device)
        w = W.scan_prefill(seqlen=L)
        stream = torch.cuda.Stream(device)
        _, calls, cfg = scan_calls(torch, ssm, W, "prefill", 1, device, stream=stream, w=w)
        del w
        ws = calls[0]._keep[-1]
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        with torch.cuda.stream(stream):
            _, call_ms, _ = timed_loop(torch, ssm, calls, 10, 2, per_launch=False)
        peak = torch.cuda.max_memory_allocated(device) - base
        E, N = cfg["dim"], cfg["d_state"]
        rows.append({"seq_len": L, "ms_per_call": round(call_ms, 4), "tokens_per_s": round(L / (call_ms * 1e-3), 1),
                     "workspace_bytes": ws_bytes, "inputs_outputs_bytes": cfg["bytes"],
                     "peak_device_bytes": int(peak), "all_states_fp32_bytes": 4 * L * E * N})
        del calls
        torch.cuda.empty_cache()
    return {"note": "batch 1, E 7680, N 16, the layer-prefill recipe; the state carried between steps stays in "
                    "registers, so memory grows with L only through the inputs, outputs and the workspace",
            "rows": rows}


def run_variants(torch, ssm, W, which, device, steps, warmup, split=0):
    """The workload with A as a model stores it and on the general path."""
    out = {}
    for v in ("log_init", "general"):
        log(f"variant: {which} {v}")
        w = make_scan_workload(W, which, v)
        stream = torch.cuda.Stream(device)
        _, calls, cfg = scan_calls(torch, ssm, W, which, 1, device, stream=stream, split=split, w=w)
        del w
        with torch.cuda.stream(stream):
            _, kmean, _ = timed_loop(torch, ssm, calls, steps, warmup)
            _, call_ms, _ = timed_loop(torch, ssm, calls, steps, warmup, per_launch=False)
        tokens = cfg["batch"] * cfg["seq_len"]
        out[v] = {"note": VARIANT_NOTES[v], "ms_per_call": round(call_ms, 4),
                  "tokens_per_s": round(tokens / (call_ms * 1e-3), 1),
                  "main_kernel_us": round(kmean * 1e3, 2),
                  "hbm_frac_of_main_kernel": round(cfg["bytes"] / (kmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "hbm_frac_of_call": round(cfg["bytes"] / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del calls
        torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (nothing here shards or "
              f"communicates across GPUs)", file=sys.stderr)
        sys.exit(2)
    import ssm_workloads as W

    which = a.only or a.workload
    # the headline workload is drawn once; the oracle baseline runs on it
    # before anything touches the GPU (its worker processes are forked)
    head_w = None
    cpu = None
    if which in ("bulk", "prefill"):
        log(f"generating the {which} workload")
        head_w = make_scan_workload(W, which)
        if not a.no_cpu and not a.only:
            log("oracle on the host CPU cores")
            cpu = cpu_baseline(head_w, WORKLOAD_NAMES[which])
            log(f"oracle: {cpu['value']} tokens/s on {cpu['cores']} cores, {cpu['single_core']['value']} on one")

    import torch
    import selective_state_space_03_amd as ssm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    ssm.lib()

    if a.only == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {a.steps} x 1 GiB device to device")
        return
    if a.only == "decode":
        graph, launches, cfg = decode_graph(torch, ssm, W, dev)
        per_call = graph_time(torch, graph, launches, a.steps)
        log(f"decode: {per_call * 1e3:.2f} us per layer-step ({launches} launches per graph, {a.steps} replays)")
        return
    if a.only == "ssd_decode":
        graph, launches, cfg = decode_graph(torch, ssm, W, dev, layers=4, ring=8, make=ssd_decode_calls)
        per_call = graph_time(torch, graph, launches, a.steps)
        log(f"ssd_decode: {per_call * 1e3:.2f} us per step ({launches} launches per graph, {a.steps} replays), "
            f"{cfg['bytes'] / (per_call * 1e-3) / 1e9:.0f} GB/s")
        return
    if a.only == "scan_bwd":
        calls, cfg = bwd_calls(torch, ssm, W, dev)
        wall, kmean, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup)
        log(f"scan_bwd: {wall:.3f} ms/step, main backward kernel {kmean * 1e3:.1f} us")
        return
    if a.only == "layer":
        calls, cfg = layer_calls(torch, ssm, W, dev)
        wall, kmean, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup)
        log(f"layer: {wall:.3f} ms/step, {kmean * 1e3:.1f} us per layer (events around the whole layer)")
        return
    if a.only in ("in_proj", "out_proj"):
        calls, cfg = gemm_calls(torch, ssm, a.only, dev)
        wall, kmean, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup)
        log(f"{a.only}: {wall:.3f} ms/step, main GEMM kernel {kmean * 1e3:.1f} us, "
            f"{cfg['flops'] / (kmean * 1e-3) / 1e12:.0f} TFLOP/s")
        return
    if a.only == "ssd":
        calls, cfg = ssd_calls(torch, ssm, W, dev)
        wall, kmean, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup)
        _, kcall, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup, per_launch=False)
        log(f"ssd: {wall:.3f} ms/step, main kernel {kmean * 1e3:.1f} us, whole call {kcall * 1e3:.1f} us")
        return
    if a.only in ("bulk_general", "prefill_general"):
        base = a.only.split("_")[0]
        w = make_scan_workload(W, base, "general")
        stream = torch.cuda.Stream(dev)
        _, calls, cfg = scan_calls(torch, ssm, W, base, 1, dev, stream=stream, split=a.split, w=w)
        with torch.cuda.stream(stream):
            _, kmean, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup)
            _, call_ms, _ = timed_loop(torch, ssm, calls, a.steps, a.warmup, per_launch=False)
        log(f"{a.only}: {call_ms:.3f} ms per call, main kernel {kmean * 1e3:.1f} us")
        return

    # rotate buffer sets so the working set exceeds the 256 MB last-level cache
    sets = 4 if which == "prefill" else 1
    log(f"uploading the {which} workload ({sets} buffer set(s))")
    stream = torch.cuda.Stream(dev)
    w, calls, cfg = scan_calls(torch, ssm, W, which, sets, dev, stream=stream, split=a.split, w=head_w)
    del head_w
    t = scan_step_timing(torch, ssm, calls, a.steps, a.warmup, stream)
    log(f"{which}: {t['graph']:.3f} ms/step (graph replay), {t['launch']:.3f} ms/step (launches), "
        f"{t['eager']:.3f} ms/step eager with per-call events, main kernel mean {t['kmean'] * 1e3:.1f} us "
        f"median {t['kmed'] * 1e3:.1f} us, whole call {t['call'] * 1e3:.1f} us")
    if a.only:
        return
    del calls, w
    torch.cuda.empty_cache()
    global COPY_GBS
    COPY_GBS = copy_rate(torch, dev)
    tokens = cfg["batch"] * cfg["seq_len"]
    wall = t["step"]
    out = {
        "metric": METRIC, "value": round(tokens / (wall * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(wall, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[which], "batch": cfg["batch"], "seq_len": cfg["seq_len"],
                   "dim": cfg["dim"], "d_state": cfg["d_state"],
                   "storage": ("bf16 u/dt/z/B/C in, bf16 y out, fp32 state" if which == "bulk"
                               else "bf16 x/z/B/C in, fp32 r, bf16 y out, fp32 state and conv cache"),
                   "A": "-(1..16) exact (the A_log = log(1..16) initialisation)",
                   "dt": ("E-wide bf16 pre-activation + bias, softplus, clip [1e-3, 0.1]" if which == "bulk"
                          else "rank-1 dt_proj of r + bias, softplus, clip [1e-3, 0.1]"),
                   "buffer_sets": sets},
        "timing": "each step one ssm_scan_fwd call; ms_per_step is the faster of graph_ms_per_step (the calls "
                  "replayed from a HIP graph) and launch_ms_per_step (the calls launched back to back from "
                  "Python); eager_ms_per_step launches each call with the library's HIP events around its "
                  "main kernel (the roofline's kernel time)",
        "graph_ms_per_step": round(t["graph"], 4), "launch_ms_per_step": round(t["launch"], 4),
        "eager_ms_per_step": round(t["eager"], 4),
        "hbm_gbps": round(cfg["bytes"] / (wall * 1e-3) / 1e9, 1),
        "hbm_frac": round(cfg["bytes"] / (wall * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "channel_steps_per_s": round(tokens * cfg["dim"] / (wall * 1e-3), 1),
        "roofline": scan_line(which, cfg, t, tokens, a.split),
        "copy_gbps": round(COPY_GBS, 1),
    }
    if not a.no_variants:
        out["variants"] = run_variants(torch, ssm, W, which, dev, max(3, a.steps // 4), 2, split=a.split)

    if not a.no_parts:
        parts = {}
        other = "bulk" if which == "prefill" else "prefill"
        log(f"part: {other} scan")
        stream2 = torch.cuda.Stream(dev)
        _, c2, cfg2 = scan_calls(torch, ssm, W, other, 4 if other == "prefill" else 1, dev, stream=stream2)
        t2 = scan_step_timing(torch, ssm, c2, 20 if other == "prefill" else 5, 2, stream2)
        tok2 = cfg2["batch"] * cfg2["seq_len"]
        parts[f"scan_{other}"] = {
            "tokens_per_s": round(tok2 / (t2["step"] * 1e-3), 1), "ms_per_call": round(t2["step"], 4),
            "hbm_gbps": round(cfg2["bytes"] / (t2["step"] * 1e-3) / 1e9, 1),
            "roofline": scan_line(other, cfg2, t2, tok2),
            "config": {k: cfg2[k] for k in ("batch", "seq_len", "dim", "d_state")}}
        del c2
        torch.cuda.empty_cache()
        if not a.no_variants:
            parts[f"scan_{other}"]["variants"] = run_variants(torch, ssm, W, other, dev, 5, 2)

        if blocked_path(which, a.split):
            log("part: the bulk call on the time-split kernels (4 segments)")
            stream5 = torch.cuda.Stream(dev)
            _, c5, cfg5 = scan_calls(torch, ssm, W, which, 1, dev, stream=stream5, split=4)
            with torch.cuda.stream(stream5):
                _, km5, _ = timed_loop(torch, ssm, c5, 5, 2)
                _, call5, _ = timed_loop(torch, ssm, c5, 5, 2, per_launch=False)
            parts["scan_bulk_time_split_4"] = {
                "note": "the same bulk call with time_split = 4: B/C packing, a summary pass over segments 0-2, "
                        "their composition, and the full pass (the library's choice below 768 channel groups)",
                "ms_per_call": round(call5, 4), "main_kernel_us": round(km5 * 1e3, 2),
                "hbm_frac_of_call": round(cfg5["bytes"] / (call5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic_of_call": call_traffic(which, 4)}
            del c5
            torch.cuda.empty_cache()

        log("part: sequence-length sweep of the layer prefill")
        parts["prefill_seqlen_sweep"] = seqlen_sweep(torch, ssm, W, dev)

        log("part: decode step (8 state sets, replayed from a HIP graph)")
        graph, launches, cfg3 = decode_graph(torch, ssm, W, dev)
        per_call = graph_time(torch, graph, launches, 8)
        parts["decode_step"] = {
            "tokens_per_s": round(cfg3["batch"] / (per_call * 1e-3), 1), "us_per_step": round(per_call * 1e3, 2),
            "roofline": roof_hbm(cfg3["bytes"], per_call, recorded_traffic("decode")),
            "timing": "HIP graph of 16 tokens x 8 layers, events around 8 replays",
            "config": {k: cfg3[k] for k in ("batch", "dim", "d_state", "layers")}}
        del graph
        torch.cuda.empty_cache()

        log("part: chunked SSD")
        c4, cfg4 = ssd_calls(torch, ssm, W, dev)
        # the main kernel from the library's events around it; the whole
        # call (segment summaries, their composition, main kernel) from
        # events around back-to-back calls
        wall4, km4, _ = timed_loop(torch, ssm, c4, 5, 1)
        _, kc4, _ = timed_loop(torch, ssm, c4, 5, 1, per_launch=False)
        r4 = roof_hbm(cfg4["bytes"], km4, recorded_traffic("ssd"))
        r4["mfma_tflops"] = round(cfg4["flops"] / (km4 * 1e-3) / 1e12, 2)
        r4["mfma_frac"] = round(r4["mfma_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)
        r4["whole_call_gbps"] = round(cfg4["bytes"] / (kc4 * 1e-3) / 1e9, 1)
        r4["whole_call_frac"] = round(cfg4["bytes"] / (kc4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        parts["chunk_scan"] = {
            "tokens_per_s": round(cfg4["seq_len"] * cfg4["batch"] / (kc4 * 1e-3), 1),
            "ms_per_call": round(kc4, 4), "main_kernel_ms": round(km4, 4), "roofline": r4,
            "config": {k: cfg4[k] for k in ("batch", "seq_len", "nheads", "headdim", "d_state", "chunk_size")}}
        del c4
        torch.cuda.empty_cache()

        log("part: SSD-form decode step (4 state sets, replayed from a HIP graph)")
        graph, launches, cfg5 = decode_graph(torch, ssm, W, dev, layers=4, ring=8, make=ssd_decode_calls)
        per_call = graph_time(torch, graph, launches, 8)
        parts["chunk_decode_step"] = {
            "tokens_per_s": round(cfg5["batch"] / (per_call * 1e-3), 1), "us_per_step": round(per_call * 1e3, 2),
            "roofline": roof_hbm(cfg5["bytes"], per_call, recorded_traffic("ssd_decode")),
            "timing": "HIP graph of 8 tokens x 4 state sets, events around 8 replays",
            "config": {k: cfg5[k] for k in ("batch", "nheads", "headdim", "ngroups", "d_state", "layers")}}
        del graph
        torch.cuda.empty_cache()

        log("part: backward of the scan stage")
        c7, cfg7 = bwd_calls(torch, ssm, W, dev)
        wall7, km7, _ = timed_loop(torch, ssm, c7, 10, 2)
        tok7 = cfg7["batch"] * cfg7["seq_len"]
        ch7 = tok7 * cfg7["dim"]
        tf7 = BWD_FLOPS_PER_CH_STEP * ch7 / (km7 * 1e-3) / 1e12
        parts["scan_backward"] = {
            "tokens_per_s": round(tok7 / (wall7 * 1e-3), 1), "ms_per_call": round(wall7, 4),
            "main_kernel_us": round(km7 * 1e3, 2),
            "roofline": {"bound": "alu", "achieved": round(tf7, 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf7 / FP32_VECTOR_PEAK_TFLOPS, 4),
                         "frac_of_unpacked": round(tf7 / (FP32_VECTOR_PEAK_TFLOPS / 2), 4),
                         "traffic": recorded_traffic("scan_bwd"),
                         "kernel": "bwd_main (the backward walk: runs of four 16-step segments per wave)",
                         "flops_per_channel_step": BWD_FLOPS_PER_CH_STEP},
            "hbm": {"algorithmic_bytes": cfg7["bytes"],
                    "whole_call_frac": round(cfg7["bytes"] / (wall7 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "config": {k: cfg7[k] for k in ("batch", "seq_len", "dim", "d_state")}}
        del c7
        torch.cuda.empty_cache()

        log("part: whole layer forward (in_proj, x_proj, scan, out_proj)")
        c6, cfg6 = layer_calls(torch, ssm, W, dev)
        wall6, km6, _ = timed_loop(torch, ssm, c6, 10, 2)
        tok6 = cfg6["batch"] * cfg6["seq_len"]
        gemms = {}
        for proj in ("in_proj", "out_proj"):
            cg, cfgg = gemm_calls(torch, ssm, proj, dev)
            _, kmg, _ = timed_loop(torch, ssm, cg, 10, 2)
            tf = cfgg["flops"] / (kmg * 1e-3) / 1e12
            gemms[proj] = {
                "kernel_us": round(kmg * 1e3, 2),
                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                             "traffic": recorded_traffic(f"gemm_{proj}")},
                "mfma_work_frac": round(cfgg["mfma_flops"] / (kmg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "config": {k: cfgg[k] for k in ("M", "K", "N", "x_dtype")}}
            del cg
        parts["layer_forward"] = {
            "tokens_per_s": round(tok6 / (wall6 * 1e-3), 1), "ms_per_call": round(wall6, 4),
            "us_per_layer": round(km6 * 1e3, 2),
            "tflops": round(cfg6["flops"] / (km6 * 1e-3) / 1e12, 1),
            "projections": gemms,
            "config": {k: cfg6[k] for k in ("batch", "seq_len", "d_model", "dim", "d_state")}}
        del c6
        torch.cuda.empty_cache()
        out["parts"] = parts

    # The pages' own figures are relative and state no hardware, precision or
    # workload: context, not targets.
    out["context"] = {
        "pages_relative_claims": [
            "up to 5x inference throughput, Mamba vs Transformer (hardware, model, batch and sequence not stated)",
            "Mamba-2 core layer 2-8x faster than Mamba's (hardware not stated)",
        ],
        "pages_absolute_numbers": None,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
