"""Benchmark: chunk-wise In-Place TTT over a 128k-token stream on one MI355X.

A step is one full pass of the hot path (target gather, up/gate GEMM + SwiGLU,
state update with snapshots, within-group scores, output GEMM) over one batch
of synthetic input, starting from a reset fast weight. Inputs are resident in
HBM before timing starts. Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--chunk C] [--no-sweep] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-MLP tokens/s per layer at d=2560/ff=9728, 128k ctx; MFMA % of peak"
WORKLOAD = "c4_4b_128k"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30  # the calibration copy reads and writes this many bytes
KERNEL_OF_PHASE = {"up_gate_swiglu": "k_a1", "update_snapshots": "k_update", "output": "k_out"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c4_4b_128k.txt")
# the sources the bf16 kernels are compiled from; the traffic summary is keyed to their hash
KERNEL_SOURCES = [os.path.join(ROOT, "chunk_wise_weight_amd", "csrc", n) for n in ("kernels_bf16.hip", "common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=256)
    ap.add_argument("--seq-len", type=int, default=None, help="override T (default: the workload's 131072)")
    ap.add_argument("--group-chunks", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the extra legs: C = 128/512/1024, update clipping at tau=1e-5, the general K=5 "
                         "target, four packed documents")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-baseline duration")
    ap.add_argument("--stack", action="store_true",
                    help="measure the 36-layer stack (B=2 x 16384 tokens, C=256) instead of the single layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of COPY_BYTES (calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--lib", default=None,
                    help="time another build of libttt.so instead of the in-tree one (same-box A/B comparisons)")
    return ap.parse_args()


def ttt_phases():
    import chunk_wise_weight_amd as ttt
    return ttt.PHASES


def algorithmic_flops(d, f, tokens):
    # per token: up/gate 4df, output 2df, update 2df
    return {"up_gate_swiglu": 4.0 * d * f * tokens, "update_snapshots": 2.0 * d * f * tokens,
            "group_scores": 0.0, "output": 2.0 * d * f * tokens, "clip_factors": 0.0}


def measured_traffic(kernel, C):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary.

    The summary holds FETCH_SIZE + WRITE_SIZE per dispatch, already scaled by
    what the same counters read for a plain copy of known size, together with
    the SHA-256 of the kernel sources they were taken on. Returns None when the
    summary is missing, covers another chunk size, or the source has changed.
    """
    import hashlib

    if not os.path.exists(TRAFFIC_FILE):
        return None
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()
    fields = {}
    for line in open(TRAFFIC_FILE):
        parts = line.split()
        if len(parts) >= 2 and not line.startswith("#"):
            fields.setdefault(parts[0], parts[1:])
    if fields.get("source_sha256", [None])[0] != sha or fields.get("chunk", [None])[0] != str(C):
        return None
    # the state update is two launches (whole rounds, then the half-tile round): one figure per call
    rows = [v for k, v in fields.items() if k == "bytes_" + kernel or k.startswith("bytes_" + kernel + "_")]
    return sum(float(r[0]) for r in rows) if rows else None


def copy_calibration():
    """One plain device-to-device copy of COPY_BYTES, for the counter calibration."""
    import torch

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def run_gpu(w, C, steps, warmup, G, clip_tau=0.0, target_conv=None, doc_starts=None):
    import numpy as np
    import torch

    import chunk_wise_weight_amd as ttt

    dt = torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)

    h = ttt.ttt_init(dev(w.W_up), dev(w.W_gate), dev(w.W_down0), C, w.eta, max_batch=w.B)
    if G:
        ttt.ttt_set_group_chunks(h, G)
    if clip_tau:
        ttt.ttt_set_clip(h, clip_tau)
    if target_conv is not None:
        ttt.ttt_set_target_conv(h, dev(target_conv[0]), dev(target_conv[1]))
    x, E = dev(w.x), dev(w.E_tgt)
    ids = torch.from_numpy(np.ascontiguousarray(w.ids)).cuda()
    y = torch.empty((w.B, w.T, w.d), dtype=dt, device="cuda")
    ttt.ttt_set_profiling(h, True)
    def forward():
        if doc_starts is None:
            ttt.ttt_forward_chunked(h, x, ids, E, y=y)
        else:
            ttt.ttt_forward_docs(h, x, ids, E, doc_starts, y=y)

    for _ in range(warmup):
        ttt.ttt_reset(h)
        forward()
    torch.cuda.synchronize()
    # a new timing window for the timed steps; the library folds event sets
    # beyond its ring of 16 into running sums, so the steps run back to back
    # with one read at the end
    ttt.ttt_set_profiling(h, True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        ttt.ttt_reset(h)
        forward()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    phase_ms = list(ttt.ttt_phase_times(h))  # the mean per call over the timed steps
    plan = ttt.ttt_plan(w.T, C, G)
    ws = ttt.ttt_workspace_bytes(h)
    ttt.ttt_destroy(h)
    del x, E, ids, y
    torch.cuda.empty_cache()
    return {"wall_s": wall, "event_ms": ev_ms, "phase_ms": phase_ms, "plan": plan,
            "workspace_bytes": ws}


def cpu_baseline(w, C, target_s):
    """The oracle as it stands, on the first S tokens of sequence 0 (a bounded sample)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    host_cpus = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = host_cpus

    def run(S):
        ids = w.ids[0, :S + 1]
        uniq, inv = np.unique(ids, return_inverse=True)
        E_s = w.E_tgt[uniq]  # the target rows this sample uses, ids remapped onto them
        t0 = time.perf_counter()
        oracle.ttt_forward_one(w.x[0, :S], inv.astype(np.int64), E_s, w.W_up, w.W_gate, w.W_down0, C, w.eta)
        return time.perf_counter() - t0

    # a short run gives the rate; the timed sample is then sized to about target_s seconds
    S = min(w.T, 4 * C)
    t = run(S)
    S = max(S, min(w.T, int(S / t * target_s) // C * C))
    t = run(S)
    # the oracle's matmuls run on the BLAS pool; everything else is one thread
    used = blas_threads if blas_threads else affinity
    return {"value": S / t, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "dtype": "f64", "blas_threads": blas_threads, "host_cpus": host_cpus, "affinity_cpus": affinity,
            "sample": f"first {S} tokens of sequence 0 ({S // C} chunks of {C}), full layer shape "
                      f"d={w.d} f={w.f}; the fp64 NumPy oracle as it stands (not the fp32 variant), target rows "
                      f"gathered to the ids used; {t:.1f} s; cores = the BLAS threads the oracle ran on"}


def run_stack(a):
    """36 independent 4B-class layers, each with its own weights, fast weights and
    synthetic input; the sequences' token stream and the target-embedding table
    are the model's, shared by every layer. One step runs all 36 layers."""
    import numpy as np
    import torch

    import chunk_wise_weight_amd as ttt
    from synth import make_config, make_inputs
    from synth.workloads import C5_LAYERS

    t0 = time.perf_counter()
    base = make_config("c5_4b_stack36")
    dt = torch.bfloat16

    def dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda", dt)

    E = dev(base.E_tgt)
    ids = torch.from_numpy(np.ascontiguousarray(base.ids)).cuda()
    layers = []
    for l in range(C5_LAYERS):
        w = base if l == 0 else make_inputs(d=base.d, f=base.f, B=base.B, T=base.T, C=base.C, eta=base.eta,
                                            dtype="bf16", vocab=1, e_std=0.02, seed=(5, l))
        h = ttt.ttt_init(dev(w.W_up), dev(w.W_gate), dev(w.W_down0), base.C, base.eta, max_batch=base.B)
        layers.append((h, dev(w.x)))
    print(f"[bench] stack of {C5_LAYERS} layers d={base.d} f={base.f} B={base.B} T={base.T} ready in "
          f"{time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    y = torch.empty((base.B, base.T, base.d), dtype=dt, device="cuda")

    def step():
        for h, x in layers:
            ttt.ttt_reset(h)
            ttt.ttt_forward_chunked(h, x, ids, E, y=y)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps
    tokens = base.B * base.T
    flops = 8.0 * base.d * base.f * tokens * C5_LAYERS
    ws = sum(ttt.ttt_workspace_bytes(h) for h, _ in layers)
    out = {
        "metric": "TTT-MLP stack tokens/s, 36 layers of d=2560/ff=9728, B=2 x 16384",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c5_4b_stack36: 36 SwiGLU MLP layers, own weights and fast W_down per sequence, "
                               "shared token stream and target table", "layers": C5_LAYERS, "d_model": base.d,
                   "d_ff": base.f, "batch": base.B, "seq_len": base.T, "chunk": base.C, "eta": base.eta,
                   "parallelism": "single GPU"},
        "layer_tokens_per_s": tokens * C5_LAYERS / (ms * 1e-3),
        "mfma_frac_stack": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "memory_gb": ws / 1e9,
    }
    for h, _ in layers:
        ttt.ttt_destroy(h)
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the fast-weight path on a single MI355X "
              "(sharding across GPUs is described in the design notes, not implemented). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from synth import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.lib:
        import chunk_wise_weight_amd.binding as binding
        binding.LIB_PATH = os.path.abspath(a.lib)
        print(f"[bench] library {binding.LIB_PATH}", file=sys.stderr, flush=True)
    if a.stack:
        run_stack(a)
        return
    t0 = time.perf_counter()
    w = make_config(WORKLOAD, C=a.chunk, T=a.seq_len)
    print(f"[bench] inputs {WORKLOAD} d={w.d} f={w.f} B={w.B} T={w.T} generated in "
          f"{time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    tokens = w.B * w.T
    flops = algorithmic_flops(w.d, w.f, tokens)
    total_flops = sum(flops.values())

    if a.copy_calibration:
        copy_calibration()
    r = run_gpu(w, a.chunk, a.steps, a.warmup, a.group_chunks)
    ms = r["event_ms"] / a.steps
    names = list(ttt_phases())
    phases = dict(zip(names, r["phase_ms"]))
    print(f"[bench] C={a.chunk}: {ms:.2f} ms/step, phases " +
          ", ".join(f"{k} {v:.3f}" for k, v in phases.items()), file=sys.stderr, flush=True)
    dom = max(("up_gate_swiglu", "update_snapshots", "output"), key=lambda k: phases[k])
    achieved = flops[dom] / (phases[dom] * 1e-3) / 1e12
    scan_ms = phases["update_snapshots"] + phases["group_scores"] + phases["output"]
    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: single SwiGLU MLP layer, fast W_down, bf16 with fp32 state",
                   "d_model": w.d, "d_ff": w.f, "batch": w.B, "seq_len": w.T, "chunk": a.chunk, "eta": w.eta,
                   "group_chunks": r["plan"]["G"], "group_tokens": r["plan"]["L"], "parallelism": "single GPU"},
        "mfma_frac_layer": total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mfma_frac_scan_gemms": (flops["update_snapshots"] + flops["output"]) / (scan_ms * 1e-3) / 1e12
        / PEAK_BF16_TFLOPS,
        "phase_ms": phases,
        # algorithmic flops over each GEMM phase's live event time (the update phase includes its snapshots)
        "phase_tflops": {k: flops[k] / (phases[k] * 1e-3) / 1e12 for k in ("up_gate_swiglu", "update_snapshots", "output")
                         if phases[k] > 0},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(KERNEL_OF_PHASE[dom], a.chunk)},
        "workspace_gb": r["workspace_bytes"] / 1e9,
    }
    def leg(key, fn):
        """Runs one optional leg; a failure is recorded in the output instead of ending the run."""
        t_leg = time.perf_counter()
        try:
            out[key] = fn()
        except Exception as e:  # noqa: BLE001 - the headline must survive any leg
            out[key] = {"error": f"{type(e).__name__}: {e}"}
            import torch
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        print(f"[bench] leg {key}: {time.perf_counter() - t_leg:.1f}s", file=sys.stderr, flush=True)

    def chunk_sweep():
        res = {}
        for Cs in (128, 512, 1024):
            if Cs == a.chunk:
                continue
            w.C = Cs
            try:
                r2 = run_gpu(w, Cs, a.steps, a.warmup, 0)
            finally:
                w.C = a.chunk
            ms2 = r2["event_ms"] / a.steps
            res[f"C{Cs}"] = {
                "tokens_per_s": tokens / (ms2 * 1e-3), "ms_per_step": ms2,
                "mfma_frac_layer": total_flops / (ms2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "group_tokens": r2["plan"]["L"], "phase_ms": dict(zip(names, r2["phase_ms"]))}
        return res

    def clip_leg():
        # the pages' long-context setting: Frobenius clipping of each chunk update at 1e-5
        r3 = run_gpu(w, a.chunk, a.steps, a.warmup, a.group_chunks, clip_tau=1e-5)
        ms3 = r3["event_ms"] / a.steps
        return {"clip_tau": 1e-5, "tokens_per_s": tokens / (ms3 * 1e-3), "ms_per_step": ms3,
                "phase_ms": dict(zip(names, r3["phase_ms"]))}

    def target_conv_leg():
        # the general target Conv1D(X0) W_target with a kernel of 5 taps (E_tgt as X0)
        from synth import make_target_conv
        r4 = run_gpu(w, a.chunk, a.steps, a.warmup, a.group_chunks,
                     target_conv=make_target_conv(w.d, 5, "bf16", seed=4))
        ms4 = r4["event_ms"] / a.steps
        return {"K": 5, "tokens_per_s": tokens / (ms4 * 1e-3), "ms_per_step": ms4,
                "phase_ms": dict(zip(names, r4["phase_ms"]))}

    def docs_leg(ndocs, clip_tau=0.0):
        # packed documents: ndocs documents of T/ndocs tokens per sequence, the state reset at each start
        starts = [[w.T // ndocs * k for k in range(1, ndocs)] for _ in range(w.B)]
        r5 = run_gpu(w, a.chunk, a.steps, a.warmup, a.group_chunks, doc_starts=starts, clip_tau=clip_tau)
        ms5 = r5["event_ms"] / a.steps
        res = {"documents_per_sequence": ndocs, "tokens_per_doc": w.T // ndocs,
               "tokens_per_s": tokens / (ms5 * 1e-3), "ms_per_step": ms5,
               "phase_ms": dict(zip(names, r5["phase_ms"]))}
        if clip_tau:
            res["clip_tau"] = clip_tau
        return res

    def shard_legs():
        # One GPU's share of the layer split over 8 GPUs (the split itself is not built): a d_ff slice of
        # 1280 (9728 is 38 tiles of 256, cut 5,5,5,5,5,5,4,4), whose y is a partial sum that a reduce-scatter
        # would finish; and a context-parallel span of T/8 tokens of the whole layer, whose ids end with the
        # next span's first token.
        import dataclasses
        fs, ts = 1280, w.T // 8
        legs = {f"dff_slice_{fs}": dataclasses.replace(w, f=fs, W_up=w.W_up[:fs], W_gate=w.W_gate[:fs],
                                                        W_down0=w.W_down0[:, :fs]),
                f"cp_span_{ts}": dataclasses.replace(w, T=ts, x=w.x[:, :ts], ids=w.ids[:, :ts + 1])}
        res = {}
        for key, ws in legs.items():
            r6 = run_gpu(ws, a.chunk, a.steps, a.warmup, a.group_chunks)
            ms6 = r6["event_ms"] / a.steps
            fl6 = 8.0 * ws.d * ws.f * ws.B * ws.T
            res[key] = {"d_ff": ws.f, "seq_len": ws.T, "ms_per_step": ms6,
                        "tokens_per_s": ws.B * ws.T / (ms6 * 1e-3),
                        "mfma_frac_layer": fl6 / (ms6 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "phase_ms": dict(zip(names, r6["phase_ms"]))}
        return res

    if not a.no_cpu_baseline:
        leg("cpu_baseline", lambda: cpu_baseline(w, a.chunk, a.cpu_seconds))
    if not a.no_sweep:
        leg("chunk_sweep", chunk_sweep)
        leg("clip_leg", clip_leg)
        leg("target_conv_leg", target_conv_leg)
        leg("docs_leg", lambda: docs_leg(4))
        leg("docs_leg_short", lambda: docs_leg(64))
        leg("docs_leg_short_clip", lambda: docs_leg(64, clip_tau=1e-5))
        leg("shard_legs", shard_legs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
