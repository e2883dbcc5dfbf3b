"""Throughput of the KV-cached attention step on one MI355X.

A step is one pass of the whole path over one batch: append the T new K/V
rows of every sequence (kvc_append), then attend the new queries over the
cache (kvc_attn_decode / kvc_attn_verify; the launch plan is host-side
inside the call). Inputs are seeded synthetic draws already resident in HBM.

value = algorithmic KV bytes per step / step time, in GB/s, where the
algorithmic bytes are the K and V rows each step must read:
sum_b seq_len_b * 2 * K * H * elem_bytes. The default workload is batched
decode (B=64, N=32, K=8, H=128, bf16, T=1, cached context U[512, 4096]).

roofline: the attention kernel alone, timed with HIP events on the stream it
is launched on: the median over 20 samples of 100 back-to-back launches, cache
replicas rotated so every launch reads from HBM rather than the 256 MB
Infinity Cache. With the default workload the same kernel figures are also
taken for the speculative-verify and paged long-context workloads
(``other_workloads``), and a plain device copy is timed as a reference
(``copy_probe``). Prints ONE JSON line. ``--gpus`` above 1 is refused: this
path runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn KV read GB/s (% of ~8 TB/s HBM peak); tokens/s per step"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix cores (MI355X published figure)
# Infinity Cache (MALL) on MI355X; cache replicas are rotated so that each
# step's reads exceed it at least twice over.
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # (the default timed region of the batched-decode step lasts over a second,
    # long enough to resolve well under 1% and to show on a utilisation probe)
    p.add_argument("--steps", type=int, default=10000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="batched_decode_b64")
    p.add_argument("--ctx", type=int, default=4096, help="cached context for layers24_b1_sweep")
    p.add_argument("--num-workgroups", type=int, default=0)
    p.add_argument("--replicas", type=int, default=0, help="cache replicas (0 = enough to defeat the MALL)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--mode", choices=("fused", "separate"), default="fused",
                   help="fused: one append_attend call per layer; separate: append, then attend")
    p.add_argument("--graph", action="store_true",
                   help="capture each replica's step in a HIP graph and replay it (launch-bound shapes)")
    p.add_argument("--others", default="auto",
                   help="comma-separated workloads whose attention kernel is also timed "
                        "(auto: the verify and paged long-context workloads with the default "
                        "workload; none: no others)")
    p.add_argument("--samples", type=int, default=20, help="kernel timing samples (median)")
    p.add_argument("--launches", type=int, default=100, help="back-to-back launches per sample")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only copy a MIB-mebibyte device buffer 10 times (known-size reference "
                        "for the HBM byte counters) and print its bandwidth")
    return p.parse_args()


def calibrate_copy(mib: int):
    """Plain device-to-device copy of a known size: the reference that scales
    FETCH_SIZE / WRITE_SIZE counters to bytes, and a copy-bandwidth figure."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "copy_GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


class Step:
    """Everything one replica of the workload needs on the GPU."""

    def __init__(self, w, prior, seed, dev, nwg, layer=None):
        import torch

        import kv_cached_gqa_attention_amd as kvc
        from workloads import draw_inputs, layout_contiguous, layout_paged, make_block_table

        self.kvc = kvc
        self.w = w
        self.inp = draw_inputs(w.B, w.T, w.N, w.K, w.H, w.dtype, prior, seed, device=dev)
        if w.layout == "paged":
            table, nb = make_block_table(seed + 7, self.inp.seq_lens, w.block_size)
            pk, pv = layout_paged(self.inp, table, nb, w.block_size, pad_value=0.0)
            self.cache = kvc.Cache(pk, pv, torch.from_numpy(table).to(dev))
        else:
            ck, cv = layout_contiguous(self.inp, pad_value=0.0)
            self.cache = kvc.Cache(ck, cv)
        # the draws' context rows are no longer needed on the device
        self.inp.ctx_k = self.inp.ctx_k[:0]
        self.inp.ctx_v = self.inp.ctx_v[:0]
        self.seq_lens = torch.from_numpy(self.inp.seq_lens.astype(np.int32)).to(dev)
        self.max_len = int(self.inp.seq_lens.max())
        self.q = self.inp.q[:, 0].contiguous() if w.T == 1 else self.inp.q
        self.out = torch.empty(self.q.shape, dtype=w.dtype, device=dev)
        self.nwg = nwg
        need = kvc.workspace_bytes(w.B, w.T, w.N, w.K, w.H, self.max_len, nwg)
        self.ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        # options: a sliding window and / or a draft-tree mask among the new tokens
        self.opts = bool(w.window or w.tree_parents)
        self.tree = None
        if w.tree_parents:
            from workloads import tree_mask_rows

            rows = tree_mask_rows(w.tree_parents).view(np.int32)  # [T, (T + 31) // 32]
            self.tree = torch.from_numpy(np.ascontiguousarray(np.tile(rows[None], (w.B, 1, 1)))).to(dev)

    def append(self):
        self.kvc.append(self.cache, self.inp.k_new, self.inp.v_new, self.seq_lens)

    def append_attend(self):
        if self.opts:
            self.kvc.attend(self.q, self.cache, self.seq_lens, self.max_len, window=self.w.window,
                            tree_mask=self.tree, k_new=self.inp.k_new, v_new=self.inp.v_new,
                            out=self.out, out_dtype=self.w.dtype, num_workgroups=self.nwg, ws=self.ws)
            return
        self.kvc.append_attend(self.q, self.inp.k_new, self.inp.v_new, self.cache, self.seq_lens,
                               self.max_len, out=self.out, out_dtype=self.w.dtype,
                               num_workgroups=self.nwg, ws=self.ws)

    def attend(self):
        if self.opts:
            self.kvc.attend(self.q, self.cache, self.seq_lens, self.max_len, window=self.w.window,
                            tree_mask=self.tree, out=self.out, out_dtype=self.w.dtype,
                            num_workgroups=self.nwg, ws=self.ws)
            return
        f = self.kvc.decode if self.w.T == 1 else self.kvc.verify
        f(self.q, self.cache, self.seq_lens, self.max_len, out=self.out, out_dtype=self.w.dtype,
          num_workgroups=self.nwg, ws=self.ws)


def source_hash() -> str:
    """Hash of the kernel sources (kv_cached_gqa_attention_amd/csrc)."""
    import hashlib

    h = hashlib.sha256()
    d = os.path.join(ROOT, "kv_cached_gqa_attention_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) from the committed
    rocprofv3 summary of this kernel and workload, or None when there is none
    or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel.replace('_kernel', '')}_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-json:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_hash") != source_hash():
                    return None
                return int(rec["fetch_bytes"] + rec["write_bytes"])
    return None


def attn_flops(w, seq_lens) -> int:
    """Algorithmic flops of one step: for every new token and query head,
    2 H for each visible key's q.k and 2 H for its p.v. Visible keys: the
    prior rows plus new tokens 0 .. t (causal inside the block), or with a
    draft tree the prior rows plus t's ancestors and t itself; with a window
    at most W keys."""
    rows = np.asarray(seq_lens, dtype=np.int64)
    t = np.arange(w.T, dtype=np.int64)
    if w.tree_parents:
        from workloads import tree_mask_rows

        own = np.array([sum(bin(int(x)).count("1") for x in row) for row in tree_mask_rows(w.tree_parents)],
                       dtype=np.int64)
    else:
        own = t + 1
    vis = rows[:, None] - w.T + own[None, :]  # keys visible to new token t
    if w.window:
        vis = np.minimum(vis, w.window)
    return int(vis.sum()) * w.N * w.H * 4


def kv_bytes(w, seq_lens) -> int:
    """Algorithmic K and V bytes of one step: every key and value row some
    new token sees, once (with a window W: the last W + T - 1 positions)."""
    rows = np.asarray(seq_lens, dtype=np.int64)
    if w.window:
        rows = np.minimum(rows, w.window + w.T - 1)
    return int(np.sum(rows)) * 2 * w.K * w.H * w.elem_bytes


def cpu_baseline(w, prior, seed, budget_s):
    """Time the CPU oracle on whole (sequence, key-value head) units of the
    same workload until ``budget_s`` seconds pass; report KV GB/s."""
    import torch

    from oracle import ancestor_words, attend
    from workloads import draw_inputs, logical_kv

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    scale = 1.0 / math.sqrt(w.H)
    G = w.N // w.K
    tree = [ancestor_words(list(w.tree_parents))] if w.tree_parents else None
    done_bytes = 0
    units = 0
    elapsed = 0.0
    n = 0
    while elapsed < budget_s:
        b = n % w.B
        one = draw_inputs(1, w.T, w.N, w.K, w.H, w.dtype, prior[b : b + 1], seed + 1000 + n, device="cpu")
        n += 1
        kb, vb = logical_kv(one, 0)
        for k in range(w.K):
            kk = kb[:, k : k + 1].double().numpy()
            vv = vb[:, k : k + 1].double().numpy()
            q = one.q[:, :, k * G : (k + 1) * G].double().numpy()
            t0 = time.perf_counter()
            attend(q, [kk], [vv], scale, window=w.window, tree_words=tree)
            elapsed += time.perf_counter() - t0
            rows = min(kk.shape[0], w.window + w.T - 1) if w.window else kk.shape[0]
            done_bytes += rows * 2 * w.H * w.elem_bytes
            units += 1
            if elapsed >= budget_s:
                break
    del torch
    return {
        "value": done_bytes / elapsed / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{units} (sequence, kv-head) units of {w.name} (prior context drawn from the same "
                  f"distribution), fp64 numpy oracle, {elapsed:.1f} s of CPU time; host has "
                  f"{os.cpu_count()} logical CPUs",
    }


def copy_probe(dev, mib=1024, samples=20):
    """A plain device-to-device copy of ``mib`` MiB (torch's copy kernel),
    median over ``samples``: the HBM read + write rate a simple streaming
    kernel reaches on this GPU, as a reference beside the 8 TB/s peak."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    times = []
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    del src, dst
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
            "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "kind": "torch device copy, median of %d" % samples}


def setup_workload(w, args, dev):
    """Replicas of one workload's step on the GPU, enough that their K/V bytes
    exceed twice the Infinity Cache (at least two)."""
    from workloads import draw_prior_lengths

    if w.prior_sweep:
        prior = np.full(w.B, args.ctx, dtype=np.int64)
    else:
        prior = draw_prior_lengths(w.seed, w.B, w.prior_lo, w.prior_hi)
    seq_lens = prior + w.T
    step_bytes = kv_bytes(w, seq_lens)
    if args.replicas > 0:
        reps = args.replicas
    else:
        reps = max(2, math.ceil(2 * MALL_BYTES / max(1, step_bytes * w.layers)))
        reps = min(reps, 4096)
    log(f"bench: {w.name} ({w.description}); KV bytes/step {step_bytes * w.layers / 1e6:.1f} MB; "
        f"{reps} replica(s) x {w.layers} layer(s)")
    steps = [[Step(w, prior, w.seed * 1000 + r * w.layers + l, dev, args.num_workgroups)
              for l in range(w.layers)] for r in range(reps)]
    return steps, prior, seq_lens, step_bytes, reps


def kernel_times(steps, one, reps, layers, stream, samples, launches):
    """Per-launch milliseconds of the attention kernel: ``samples`` samples,
    each ``launches`` back-to-back steps between two HIP events recorded on
    the launch stream, divided by the launches (and layers) it holds."""
    import torch

    for i in range(reps):
        for s in steps[i]:
            one(s)
    torch.cuda.synchronize()
    out = []
    k = 0
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            for s in steps[k % reps]:
                one(s)
            k += 1
        e1.record(stream)
        e1.synchronize()
        out.append(e0.elapsed_time(e1) / (launches * layers))
    return out


def roofline_of(w, kernel, seq_lens, step_bytes, times_ms, copy):
    """The roofline object of one workload's attention kernel from its
    per-launch time samples."""
    attn_ms = float(np.median(times_ms))
    achieved = step_bytes / (attn_ms * 1e-3) / 1e9
    step_flops = attn_flops(w, seq_lens)
    # bound: the matrix cores where the step's flops per K/V byte exceed their
    # balance against HBM (a chunk of prefill), else HBM
    mfma_bound = step_flops / step_bytes > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    r = {
        "kernel": kernel,
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": profiled_traffic(kernel, w.name),
        "launch_ms": round(attn_ms, 5),
        "launch_ms_min": round(float(np.min(times_ms)), 5),
        "launch_ms_max": round(float(np.max(times_ms)), 5),
        "timing": f"median of {len(times_ms)} samples (HIP events on the launch stream)",
        "bytes_per_launch": step_bytes,
    }
    if copy:
        r["pct_of_copy_probe"] = round(100 * achieved / copy["GBps_read_plus_write"], 2)
    tflops = step_flops / (attn_ms * 1e-3) / 1e12
    if kernel != "attn_valu_kernel" and not mfma_bound:
        # a matrix-core kernel bound by HBM: its matrix-core use beside the
        # HBM figure (algorithmic flops over the dense bf16/fp16 peak)
        r.update({"flops_per_launch": step_flops, "mfma_tflops": round(tflops, 2),
                  "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4)})
    if mfma_bound:
        r.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                  "flops_per_launch": step_flops, "hbm_GBps": round(achieved, 2)})
    return r


def plan_kernel(w, seq_lens, nwg):
    import kv_cached_gqa_attention_amd as kvc

    return kvc.plan_kernel(w.B, w.T, w.N, w.K, w.H, int(np.max(seq_lens)), nwg)


def other_workload(name, args, dev, stream, copy):
    """Kernel-only figures of another workload (same timing as the main one)."""
    from workloads import get_workload

    w = get_workload(name)
    steps, prior, seq_lens, step_bytes, reps = setup_workload(w, args, dev)
    kernel = plan_kernel(w, seq_lens, args.num_workgroups)
    times = kernel_times(steps, lambda s: s.append_attend(), reps, w.layers, stream, args.samples,
                         args.launches)
    r = roofline_of(w, kernel, seq_lens, step_bytes, times, copy)
    del steps
    return {"workload": w.name, "description": w.description, "replicas": reps,
            "mean_seq_len": float(np.mean(seq_lens)),
            "tokens_per_s": round(w.B * w.T / (r["launch_ms"] * 1e-3), 1), "roofline": r}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch

    from workloads import get_workload

    w = get_workload(args.workload)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    copy = copy_probe(dev)
    log(f"bench: copy probe {copy['GBps_read_plus_write']} GB/s read+write")
    steps, prior, seq_lens, step_bytes, reps = setup_workload(w, args, dev)
    layers = w.layers
    torch.cuda.synchronize()

    def eager_step(i):
        for s in steps[i % reps]:
            if args.mode == "fused":
                s.append_attend()
            else:
                s.append()
                s.attend()

    # The step is the same work either way; with --graph each replica's step
    # is captured once (after an eager warm-up) and replayed.
    graphs = None
    if args.graph:
        for i in range(reps):
            eager_step(i)
        torch.cuda.synchronize()
        graphs = []
        side = torch.cuda.Stream(dev)
        for i in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                eager_step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % reps].replay()
        else:
            eager_step(i)

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Attention kernel alone: back-to-back launches between two HIP events on
    # the stream the kernel runs on (torch's current stream is the one handed
    # to the library). The dominant kernel is the fused call's attention
    # kernel (its appends rewrite the same rows), or the attention kernel of
    # the separate form.
    one = (lambda s: s.append_attend()) if args.mode == "fused" else (lambda s: s.attend())
    times = kernel_times(steps, one, reps, layers, stream, args.samples, args.launches)
    kernel = plan_kernel(w, seq_lens, args.num_workgroups)
    roof = roofline_of(w, kernel, seq_lens, step_bytes, times, copy)

    value = step_bytes * layers / (ms_per_step * 1e-3) / 1e9
    tokens = w.B * w.T
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name(),
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "batch": w.B,
            "query_tokens": w.T,
            "q_heads": w.N,
            "kv_heads": w.K,
            "head_dim": w.H,
            "layers": layers,
            "kv_bytes_per_step": step_bytes * layers,
            "mean_seq_len": float(np.mean(seq_lens)),
            "replicas": reps,
            "mode": args.mode + (" + graph" if args.graph else ""),
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "attention_steps_per_s": round(1e3 / ms_per_step, 1),
        "roofline": roof,
        "copy_probe": copy,
    }
    del steps, graphs
    torch.cuda.synchronize()
    others = args.others
    if others == "auto":
        others = "spec_verify_b32_t5,paged_long_b8" if w.name == "batched_decode_b64" else "none"
    if others != "none":
        torch.cuda.empty_cache()
        result["other_workloads"] = []
        for name in [x for x in others.split(",") if x]:
            result["other_workloads"].append(other_workload(name, args, dev, stream, copy))
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, prior, w.seed, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
