"""Benchmark of the mLSTM cell forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one chunkwise forward pass (mlstm_fwd_chunkwise) over the
7B-layer-shaped prefill workload: B=8 H=8 T=4096 d_qk=256 d_v=512 chunk=64,
bf16 I/O, float32 state, synthetic seeded inputs already resident in HBM.
`value` is prefill tokens/s (B*T per step).  The same JSON line also carries
the decode workload (B=256 H=8, 1024 consecutive in-place mlstm_step calls),
the long-context prefill (B=1 H=8 T=65536 chunk=128) and the backward pass
(mlstm_bwd_chunkwise at B=4 H=4 T=1024 d=64 float32), each with its own
roofline, and the float64 oracle timed on the host cores over a bounded
sample (`cpu_baseline`).

Kernel times come from HIP events recorded on the stream the library
launches on (torch's current stream), one before every timed step and one
after the last: `ms_per_step` is the whole span over the K steps divided by
K (the mean), `ms_per_step_median` the median of the per-step spans.  Before
the warmup steps, whatever --warmup is, the prefill step runs untimed for a
fixed stretch of GPU time (--settle-ms, default 300 ms), so that the clock
has left the low state it sits in after the seconds of host-side input
generation: without it the first timed steps ran about 25% slower on the
7B-layer prefill.  Rooflines use algorithmic work:
  prefill flops per token-head  (L+1)(d_qk+d_v) + 4 d_qk d_v + 4 d_qk
  prefill bytes per token-head  2(2 d_qk + 2 d_v) + 2 d_v + 8   (bf16 q,k,v,o~ in, h out, f32 gates)
  decode bytes per pair-step    8(d_qk d_v + d_qk + 1) + 2(2 d_qk + 2 d_v) + 2 d_v + 8
                                (state read + written, bf16 q,k,v,o~ in, h out, f32 gates)
against MI355X peaks: bf16 dense MFMA 2516.6 TFLOP/s, HBM 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3  # fp32 vector peak of the chip (the unpacked FMA rate is half of it)
BWD_KERNELS = "bwd_ckpt_kernel + bwd_a_kernel + bwd_b_kernel + bwd_c_kernel + bwd_d_kernel"
METRIC = "mLSTM prefill tokens/s + %MFMA peak; decode step state GB/s + %HBM peak"
PREFILL_KERNEL = "mlstm_ws_kernel<256> (role-split chunkwise forward, one launch per step)"
CPU_THREADS_MAX = 16  # host cores that go with one GPU


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_work(w, L=None):
    """Algorithmic flops and bytes of one prefill call; flops are counted at
    chunk L (the workload's chunk unless given)."""
    L = w.chunk if L is None else L
    dk, dv = w.d_qk, w.d_v
    th = w.B * w.H * w.T
    flops = th * ((L + 1) * (dk + dv) + 4 * dk * dv + 4 * dk)
    io_bytes = th * (2 * (2 * dk + 2 * dv) + 2 * dv + 8)
    state_bytes = w.B * w.H * (dk * dv + dk + 1) * 4  # final state written
    return flops, io_bytes + state_bytes


def decode_work(w):
    """Bytes of one decode step: the state read and written (float32), and
    q, k, v, o~ read, h written (bf16), the two float32 gates read."""
    dk, dv = w.d_qk, w.d_v
    pairs = w.B * w.H
    state = pairs * 8 * (dk * dv + dk + 1)
    io = pairs * (2 * (2 * dk + 2 * dv) + 2 * dv + 8)
    return state, state + io


def traffic_record(name):
    """Measured HBM bytes per launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    from xlstm_mlstm_matrix_amd.rocprof_summary import src_hash
    if rec.get("kernel_src_sha") != src_hash(name):
        return None
    return rec.get("bytes_per_launch")


def time_steps(torch, run, steps):
    """Run `run` exactly `steps` times back to back between two device
    synchronisations, with a HIP event before every step and after the last
    (events on the stream the library launches on).  Returns (mean, median)
    milliseconds per step: the mean is the whole span over the steps, the
    median that of the per-step spans."""
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record(st)
        run()
    ev[steps].record(st)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    total = ev[0].elapsed_time(ev[steps])
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return total / steps, median


def settle_clock(torch, run, settle_ms):
    """Untimed phase of fixed duration before any warmup: runs the step until
    `settle_ms` of GPU time has passed, so that the clock has left its idle
    state whatever --warmup is.  Returns (milliseconds spent, steps run)."""
    spent, n, batch = 0.0, 0, 1
    while spent < settle_ms:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream())
        for _ in range(batch):
            run()
        b.record(torch.cuda.current_stream())
        b.synchronize()
        spent += a.elapsed_time(b)
        n += batch
        batch = min(batch * 2, 256)
    return spent, n


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record(self.torch.cuda.current_stream())
        return self

    def __exit__(self, *exc):
        self.b.record(self.torch.cuda.current_stream())
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def bench_prefill(torch, I, binding, name, steps, warmup, variant="auto", settle_ms=0.0):
    w = I.workload(name)
    t0 = time.time()
    d = I.gen_prefill(w, threads=16)
    g = {k: (v.cuda().reshape(w.B, w.H, *v.shape[1:]) if v is not None else None) for k, v in d.items()}
    del d
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s")
    args = [g[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    h = torch.empty((w.B, w.H, w.T, w.d_v), dtype=args[0].dtype, device="cuda")
    C = torch.empty((w.B, w.H, w.d_qk, w.d_v), device="cuda")
    n = torch.empty((w.B, w.H, w.d_qk), device="cuda")
    m = torch.empty((w.B, w.H), device="cuda")
    io = binding.BF16 if w.io == "bf16" else binding.F32
    ws = torch.empty(max(1, binding.workspace_size(w.B, w.H, w.T, w.d_qk, w.d_v, w.chunk, io, variant)),
                     dtype=torch.uint8, device="cuda")

    def run():
        binding.fwd_chunkwise(*args, chunk=w.chunk, variant=variant, h=h, C_T=C, n_T=n, m_T=m,
                              workspace=ws)

    settle = settle_clock(torch, run, settle_ms) if settle_ms > 0 else (0.0, 0)
    for _ in range(warmup):
        run()
    ms, med = time_steps(torch, run, steps)
    kc, _ = binding.schedule(w.B, w.H, w.T, w.d_qk, w.d_v, w.chunk, io, variant)
    flops, nbytes = prefill_work(w)
    flops_kc, _ = prefill_work(w, L=kc)
    tokens = w.B * w.T
    log(f"{name}: {ms:.4f} ms/step (median {med:.4f}; clock settled over {settle[0]:.0f} ms, "
        f"{settle[1]} steps), {tokens / ms * 1e3:.3e} tokens/s, {flops / ms / 1e9:.1f} TFLOP/s, "
        f"{nbytes / ms / 1e6:.0f} GB/s")
    return dict(w=w, ms=ms, median_ms=med, flops=flops, flops_kernel_chunk=flops_kc, kernel_chunk=kc,
                bytes=nbytes, settle_ms=settle[0], settle_steps=settle[1], keep=(g, h, C, n, m))


def bench_decode(torch, I, binding, warmup_passes=1, nsteps=None):
    w = I.workload("decode_bf16")
    if nsteps:
        w = I.workload("decode_bf16", T=nsteps)
    t0 = time.time()
    C0, n0, m0 = (x.cuda() for x in I.gen_decode_state(w, threads=16))
    steps = {}
    chunk = 128
    parts = {k: [] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")}
    for s0 in range(0, w.T, chunk):
        st = I.gen_decode_steps(w, range(s0, min(w.T, s0 + chunk)), threads=16)
        for k in parts:
            parts[k].append(st[k].cuda())
    steps = {k: torch.cat(v) for k, v in parts.items()}
    log(f"decode: inputs ready in {time.time() - t0:.1f}s")
    C, n, m = C0.clone(), n0.clone(), m0.clone()
    h = torch.empty((w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
    keys = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    # one workspace (scratch of the row-split kernel) for the whole run
    ws = binding.step_workspace(w.B, w.H, w.d_qk, w.d_v, torch.bfloat16, "cuda")

    def one_pass():
        for t in range(w.T):
            binding.step(*(steps[k][t] for k in keys), C, n, m, h=h, C_out=C, n_out=n, m_out=m,
                         workspace=ws)

    for _ in range(warmup_passes):
        one_pass()
    C.copy_(C0); n.copy_(n0); m.copy_(m0)
    with Timer(torch) as tm:
        one_pass()
    ms = tm.ms / w.T
    # a second pass with an event around every step: the per-step median
    it = iter(range(w.T))

    def one_step():
        t = next(it)
        binding.step(*(steps[k][t] for k in keys), C, n, m, h=h, C_out=C, n_out=n, m_out=m, workspace=ws)

    _, med = time_steps(torch, one_step, w.T)
    state_bytes, total_bytes = decode_work(w)
    log(f"decode: {ms:.4f} ms/step (median {med:.4f}), state {state_bytes / ms / 1e6:.0f} GB/s, "
        f"total {total_bytes / ms / 1e6:.0f} GB/s, {w.B / ms * 1e3:.3e} tokens/s")
    return w, ms, med, state_bytes, total_bytes


def backward_work(w, L=32):
    """Algorithmic flops of the chunkwise backward (checkpoint pass included):
    per token-head 6 d_qk d_v multiply-adds (the recomputed read-out, C' a,
    G* v, G*^T k, the carried-gradient update and the checkpoint pass's state
    update) plus 3 (d_qk + d_v) per causal partner ((L + 1) / 2 on average:
    S, a.v, P V, P~ K, P~^T Q, P^T A), 2 flops each."""
    th = w.B * w.H * w.T
    return th * 2 * (6 * w.d_qk * w.d_v + 1.5 * (L + 1) * (w.d_qk + w.d_v))


def bench_backward(torch, I, binding, steps, warmup, name="small_f32"):
    w = I.workload(name)
    d = I.gen_prefill(w, threads=16)
    g = {k: (v.cuda().reshape(w.B, w.H, *v.shape[1:]) if v is not None else None) for k, v in d.items()}
    del d
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    dh = torch.randn((w.B, w.H, w.T, w.d_v), generator=torch.Generator().manual_seed(7)).to(io_t).cuda()
    args = [g[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")] + [dh, g["C0"], g["n0"], g["m0"]]
    nbytes = binding.bwd_workspace_size(w.B, w.H, w.T, w.d_qk, w.d_v, 32,
                                        binding.BF16 if w.io == "bf16" else binding.F32)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run():
        binding.bwd_chunkwise(*args, chunk=32, state_grad=True, workspace=ws)

    for _ in range(warmup):
        run()
    with Timer(torch) as tm:
        for _ in range(steps):
            run()
    ms = tm.ms / steps
    fl = backward_work(w)
    log(f"backward {w.name}: {ms:.3f} ms/step, {fl / ms / 1e9:.2f} TFLOP/s")
    return w, ms, fl


def layer_work(w):
    """Algorithmic flops of one layer call: the projection GEMMs (2 flops per
    multiply-add, every output of q, k, v, o~ and the two gates) plus the
    cell's per-token-head flops (as for the prefill line)."""
    BT = w.B * w.T
    proj = 2 * BT * w.d_model * w.H * (2 * w.d_qk + 2 * w.d_v + 2)
    cell = BT * w.H * ((w.chunk + 1) * (w.d_qk + w.d_v) + 4 * w.d_qk * w.d_v + 4 * w.d_qk)
    return proj, cell


def bench_layer(torch, I, binding, steps, warmup):
    w = I.layer_workload("layer_7b_bf16")
    t0 = time.time()
    d = I.gen_layer(w, threads=16)
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    del d
    log(f"layer: inputs ready in {time.time() - t0:.1f}s")
    names = ("x", "W_q", "W_k", "W_v", "W_o", "W_i", "W_f", "b_q", "b_k", "b_v", "b_o", "b_i", "b_f")
    ws = torch.empty(binding.layer_workspace_size(w.B, w.T, w.d_model, w.H, w.d_qk, w.d_v, w.chunk,
                                                  binding.BF16), dtype=torch.uint8, device="cuda")

    def run():
        binding.layer_fwd(*(g[k] for k in names), chunk=w.chunk, return_state=True, workspace=ws)

    for _ in range(warmup):
        run()
    with Timer(torch) as tm:
        for _ in range(steps):
            run()
    ms = tm.ms / steps
    proj, cell = layer_work(w)
    log(f"layer {w.name}: {ms:.3f} ms/step, {(proj + cell) / ms / 1e9:.1f} TFLOP/s "
        f"({proj / 1e12:.2f} TFLOP projections + {cell / 1e12:.3f} TFLOP cell)")
    return w, ms, proj, cell


def slstm_work(w):
    """Algorithmic flops of one sLSTM call: per token and group, the memory
    mixing (4 matrix-vector products d x d, 2 flops per multiply-add) and
    about 12 flops per cell for the gates and the update (exp, tanh and the
    sigmoid counted as one each)."""
    return w.B * w.H * w.T * (8 * w.d * w.d + 12 * w.d)


def bench_slstm(torch, I, binding, steps, warmup):
    w = I.slstm_workload("slstm_bf16")
    d = I.gen_slstm(w, threads=16)
    gx, R = d["gx"].cuda(), d["R"].cuda()
    h = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.slstm_fwd(gx, R, return_state=False, h=h)

    for _ in range(warmup):
        run()
    with Timer(torch) as tm:
        for _ in range(steps):
            run()
    ms = tm.ms / steps
    fl = slstm_work(w)
    log(f"slstm {w.name}: {ms:.3f} ms/call, {w.B * w.T / ms * 1e3:.3e} tokens/s, "
        f"{ms * 1e3 / w.T:.3f} us per sequential step")
    return w, ms, fl


def cpu_baseline(I, pairs_sample):
    """The float64 oracle on the host cores over a bounded sample of the
    prefill workload: `pairs_sample` (b, h) pairs, full sequence each."""
    import oracle
    w = I.workload("prefill_7b_bf16")
    d = I.gen_prefill(w, pairs=pairs_sample, threads=16)
    host_cores = len(os.sched_getaffinity(0))
    threads = min(host_cores, CPU_THREADS_MAX, len(pairs_sample))
    orc = oracle.load()
    t0 = time.time()
    orc.forward(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], threads=threads)
    dt = time.time() - t0
    frac = len(pairs_sample) / (w.B * w.H)
    tokens_per_s = (w.B * w.T) * frac / dt   # the sample's share of the workload's tokens
    log(f"cpu oracle: {len(pairs_sample)} pairs x {w.T} tokens in {dt:.2f}s on {threads} threads")
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "host_cores": host_cores,
            "threads_cap": CPU_THREADS_MAX, "kind": "oracle",
            "sample": f"{len(pairs_sample)} of {w.B * w.H} (batch, head) pairs of the 7B-layer prefill "
                      f"workload, full T={w.T} each, float64 sequential recurrence, OpenMP over pairs; "
                      f"rate = sampled tokens x (pairs sampled / all pairs) / wall time "
                      f"({dt:.2f} s wall)",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed GPU time spent running the prefill step before its warmup, "
                         "whatever --warmup is, so the timed steps run at the settled clock")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-slstm", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 7B prefill line (profiling runs of the other workloads)")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="decode steps per pass (default: the workload's 1024)")
    ap.add_argument("--cpu-pairs", type=int, default=64)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also stream 1 GiB through a plain elementwise kernel (torch.neg: "
                         "1 GiB read, 1 GiB written), the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the mLSTM cells are "
              "independent per (batch, head) and would shard across GPUs without any exchange, "
              "but no multi-GPU launcher is implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    from xlstm_mlstm_matrix_amd import binding, inputs as I
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy probe: 3 x 1 GiB streamed (neg)")
        del src, dst

    if args.no_prefill:
        w = I.workload("prefill_7b_bf16")
        r = dict(w=w, ms=float("nan"), median_ms=float("nan"), flops=float("nan"),
                 flops_kernel_chunk=float("nan"), kernel_chunk=w.chunk, bytes=float("nan"),
                 settle_ms=0.0, settle_steps=0)
    else:
        r = bench_prefill(torch, I, binding, "prefill_7b_bf16", args.steps, args.warmup,
                          settle_ms=args.settle_ms)
        r.pop("keep")
        torch.cuda.empty_cache()
    w, ms, flops, nbytes = r["w"], r["ms"], r["flops"], r["bytes"]
    tflops = flops / ms / 1e9
    gbs = nbytes / ms / 1e6
    kc, nseg = binding.schedule(w.B, w.H, w.T, w.d_qk, w.d_v, w.chunk, binding.BF16)
    rec = {
        "metric": METRIC,
        "value": w.B * w.T / ms * 1e3,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": r["median_ms"],
        "clock_settle": {"ms": r["settle_ms"], "steps": r["settle_steps"]},
        # the headline's two fractions side by side: algorithmic flops over the
        # bf16 MFMA peak, algorithmic bytes over the HBM peak (the kernel is
        # bound by HBM: 136 flop per byte, below the ridge)
        "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "hbm_frac": gbs / PEAK_HBM_GBS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, distributions of the workload spec)",
        "config": {"workload": "prefill B=8 H=8 T=4096 d_qk=256 d_v=512 chunk=64 bf16 I/O fp32 state",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "d_qk": w.d_qk, "d_v": w.d_v,
                   "chunk": w.chunk, "kernel_chunk": kc, "segments": nseg,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": traffic_record("prefill_7b"),
                     "mfma_achieved_tflops": tflops, "mfma_peak_tflops": PEAK_BF16_TFLOPS,
                     "mfma_frac": tflops / PEAK_BF16_TFLOPS,
                     "kernel": PREFILL_KERNEL,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes},
    }

    if not args.no_long:
        try:
            rl = bench_prefill(torch, I, binding, "prefill_long_bf16", max(3, args.steps // 4),
                               max(1, args.warmup // 4), settle_ms=min(args.settle_ms, 100.0))
            rl.pop("keep")
            torch.cuda.empty_cache()
            wl, msl = rl["w"], rl["ms"]
            kcl, nsl = binding.schedule(wl.B, wl.H, wl.T, wl.d_qk, wl.d_v, wl.chunk, binding.BF16)
            rec["long_context"] = {
                "workload": "prefill B=1 H=8 T=65536 d_qk=256 d_v=512 chunk=128 bf16 I/O fp32 state, "
                            "final state returned",
                "kernel_chunk": kcl, "segments": nsl,
                "ms_per_step": msl, "ms_per_step_median": rl["median_ms"],
                "tokens_per_s": wl.B * wl.T / msl * 1e3,
                "mfma_frac": rl["flops"] / msl / 1e9 / PEAK_BF16_TFLOPS,
                "mfma_frac_at_kernel_chunk": rl["flops_kernel_chunk"] / msl / 1e9 / PEAK_BF16_TFLOPS,
                "flops_note": f"mfma_frac counts the intra-chunk flops at the requested chunk "
                              f"({wl.chunk}); mfma_frac_at_kernel_chunk at the executed one ({kcl})",
                "hbm_frac": rl["bytes"] / msl / 1e6 / PEAK_HBM_GBS}
        except Exception as e:  # reported, not hidden
            rec["long_context"] = {"error": str(e)}
            log(f"long context: {e}")

    if not args.no_decode:
        wd, msd, medd, sb, tb = bench_decode(torch, I, binding, nsteps=args.decode_steps or None)
        rec["decode"] = {
            "workload": "decode B=256 H=8 d_qk=256 d_v=512, 1024 in-place mlstm_step calls, bf16 I/O fp32 state",
            "ms_per_step": msd, "ms_per_step_median": medd, "tokens_per_s": wd.B / msd * 1e3,
            "state_GBs": sb / msd / 1e6,
            "roofline": {"bound": "hbm", "achieved": tb / msd / 1e6, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": tb / msd / 1e6 / PEAK_HBM_GBS, "traffic": traffic_record("decode"),
                         "kernel": "mlstm_step_rows_kernel + mlstm_step_finish_kernel (row split, two launches per step)",
                         "algorithmic_bytes_per_step": tb}}

    if not args.no_backward:
        wb, msb, flb = bench_backward(torch, I, binding, max(3, args.steps // 4), max(1, args.warmup // 4))
        rec["backward"] = {
            "workload": "backward B=4 H=4 T=1024 d_qk=d_v=64 float32 I/O, initial-state gradients "
                        "(checkpoint pass + chunk-parallel passes and column-block scans, 32-token chunks)",
            "ms_per_step": msb, "tokens_per_s": wb.B * wb.T / msb * 1e3,
            "roofline": {"bound": "alu", "achieved": flb / msb / 1e9, "peak": PEAK_FP32_TFLOPS,
                         "unit": "TFLOP/s", "frac": flb / msb / 1e9 / PEAK_FP32_TFLOPS, "traffic": None,
                         "kernel": BWD_KERNELS,
                         "algorithmic_flops_per_launch": flb}}
        wb7, msb7, flb7 = bench_backward(torch, I, binding, 2, 1, name="prefill_7b_bf16")
        rec["backward_7b"] = {
            "workload": "backward B=8 H=8 T=4096 d_qk=256 d_v=512 bf16 I/O, zero state "
                        "(checkpoint pass + chunk-parallel passes and column-block scans, 32-token chunks)",
            "ms_per_step": msb7, "tokens_per_s": wb7.B * wb7.T / msb7 * 1e3,
            "roofline": {"bound": "alu", "achieved": flb7 / msb7 / 1e9, "peak": PEAK_FP32_TFLOPS,
                         "unit": "TFLOP/s", "frac": flb7 / msb7 / 1e9 / PEAK_FP32_TFLOPS,
                         "traffic": traffic_record("backward_7b"),
                         "traffic_note": "HBM bytes per call summed over bwd_ckpt/a/b/c_kernel<bf16> "
                                         "(bwd_d_kernel moves a few KB)",
                         "kernel": BWD_KERNELS,
                         "algorithmic_flops_per_launch": flb7}}

    if not args.no_layer:
        wl, msl_, projf, cellf = bench_layer(torch, I, binding, max(3, args.steps // 10),
                                             max(2, args.warmup // 20))
        rec["layer"] = {
            "workload": "mLSTM layer forward B=8 T=4096 d_model=4096 H=8 d_qk=256 d_v=512 chunk=64 bf16: "
                        "all-heads projections (hipBLASLt) + gate bias + chunkwise cell on strided rows",
            "ms_per_step": msl_, "tokens_per_s": wl.B * wl.T / msl_ * 1e3,
            "roofline": {"bound": "mfma", "achieved": (projf + cellf) / msl_ / 1e9,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": (projf + cellf) / msl_ / 1e9 / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "hipBLASLt GEMMs (q, k, v, o~ over all heads + one gate GEMM) + "
                                   "gate_bias_kernel + mlstm_ws_kernel",
                         "algorithmic_flops_per_step": projf + cellf,
                         "projection_flops": projf, "cell_flops": cellf}}

    if not args.no_slstm:
        ws_, mss, fls = bench_slstm(torch, I, binding, 3, 1)
        rec["slstm"] = {
            "workload": "sLSTM cell forward B=16 H=8 T=4096 d=128 bf16 I/O, zero state "
                        "(sequential in T: one workgroup per (batch, head) group)",
            "ms_per_step": mss, "tokens_per_s": ws_.B * ws_.T / mss * 1e3,
            "us_per_sequential_step": mss * 1e3 / ws_.T,
            "roofline": {"bound": "alu", "achieved": fls / mss / 1e9, "peak": PEAK_FP32_TFLOPS,
                         "unit": "TFLOP/s", "frac": fls / mss / 1e9 / PEAK_FP32_TFLOPS, "traffic": None,
                         "kernel": "slstm_kernel<bf16, 128>", "algorithmic_flops_per_launch": fls}}

    if not args.no_cpu:
        Pn = max(1, args.cpu_pairs)
        sample = [(p // 8, p % 8) for p in range(0, 64, max(1, 64 // Pn))][:Pn]
        log(f"cpu oracle: {len(sample)} pairs")
        rec["cpu_baseline"] = cpu_baseline(I, sample)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
