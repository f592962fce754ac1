#!/usr/bin/env python3
"""Benchmark of the HiSA hot path on one MI355X.

A step is one layer's pass of the whole path over one batch of synthetic
input: selection (gate, block means, coarse top-Kb, fine top-k, or the flat
scan) followed by the sparse local + pooled attention that consumes it.  The
default workload is one V4-Flash-shaped decode step at Np = 16384 pooled keys
(B = 1, 64 x 128 bf16 indexer, top-512 of blocks of 64, 64 heads x 512, window
128, sinks).  Inputs are resident in HBM before timing starts; R copies of the
inputs are cycled so that each step reads data the 256 MiB Infinity Cache does
not hold.

Prints ONE JSON line: rows/s (B*L / step time), us per layer, step GB/s, the
roofline of the dominant kernel (its algorithmic bytes or flops per launch over
its average duration from HIP events on its stream), and the CPU oracle timed
on the host's cores on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-query rows/sec + µs/layer decode at Np=16K; achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_DEFEAT_BYTES = 640 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="v4flash_decode_np16384")
    ap.add_argument("--graph", action="store_true", help="replay the timed steps from a captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (scale for the HBM byte counters)")
    return ap.parse_args()


def kernel_sources_sha():
    """Hash of the kernel sources and the build script (its compiler flags),
    to tell whether stored counters still apply."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "top_kv_indexer_amd")
    csrc = os.path.join(pkg, "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))] + [os.path.join(pkg, "build.py")]
    for path in files:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel reading), or
    None when no summary exists or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != kernel_sources_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def algorithmic(w, x, unique_kv_rows=None, flat_seqs=None):
    """Compulsory bytes / flops per kernel family for one step of workload w.
    Bytes: every input read once and every output written once; flops: the
    method's own multiply-adds (x2).  unique_kv_rows: distinct KV rows the
    attention reads in the step (each counted once)."""
    B, L = w.B, w.L
    Np = [int(n) for n in x["Np"]]
    rows = B * L
    bf = 2 if w.bf16 else 4
    idx_q = rows * w.H_i * w.D_i * bf + rows * w.H_i * 4
    keys = sum(Np) * w.D_i * bf
    kI = w.topk
    n_local = min(w.window, int(x["Wl_cap"]))
    if unique_kv_rows is None:
        unique_kv_rows = rows * (kI + n_local)
    attn_bytes = unique_kv_rows * w.Dk * bf + rows * w.H * w.Dk * bf + rows * w.H * w.Dv * bf \
        + rows * kI * 4 + (w.H * 4 if w.sinks else 0)
    attn_flops = rows * (kI + n_local) * w.H * (w.Dk + w.Dv) * 2
    nb = [n // w.index_block for n in Np] if w.index_block else [0] * B
    flat = list(range(B)) if flat_seqs is None else [b for b in range(B) if flat_seqs[b]]
    C = w.index_keep * w.index_block
    return {
        "decode_scan": {"bytes": keys + idx_q, "flops": sum(Np) * w.H_i * w.D_i * 2},
        "decode_select": {"bytes": rows * kI * 4, "flops": 0},
        "decode_scan_select": {"bytes": keys + idx_q + rows * kI * 4, "flops": sum(Np) * w.H_i * w.D_i * 2},
        "attention": {"bytes": attn_bytes, "flops": attn_flops},
        "attention_merge": {"bytes": rows * w.H * w.Dv * bf, "flops": 0},
        "block_mean": {"bytes": keys, "flops": 0},
        "coarse": {"bytes": idx_q, "flops": L * sum(nb) * w.H_i * w.D_i * 2},
        "fine": {"bytes": idx_q + rows * kI * 4, "flops": rows * C * w.H_i * w.D_i * 2},
        # the flat scan scores only the sequences on the flat path
        "flat_scores": {"bytes": sum(Np[b] for b in flat) * w.D_i * bf + len(flat) * L * (w.H_i * w.D_i * bf + w.H_i * 4),
                        "flops": sum(sum(min(Np[b], (int(x["t0"][b]) + j + 1) // w.ratio) for j in range(L))
                                     for b in flat) * w.H_i * w.D_i * 2},
        "topk_rows": {"bytes": len(flat) * L * kI * 4, "flops": 0},
        "select_rows": {"bytes": idx_q + rows * kI * 4,
                        "flops": L * sum(nb) * w.H_i * w.D_i * 2 + rows * C * w.H_i * w.D_i * 2},
    }


def rate(a, seconds):
    """Roofline position of one launch with algorithmic cost `a` that took
    `seconds`: bf16 MFMA-bound when its flops take longer at peak than its
    bytes at HBM peak, else HBM-bound."""
    if a["flops"] / BF16_PEAK_TFLOPS / 1e12 > a["bytes"] / HBM_PEAK_GBPS / 1e9:
        ach = a["flops"] / seconds / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    ach = a["bytes"] / seconds / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4)}


def cpu_baseline(w, x, seconds):
    """The oracle (as it stands) on the host: threads each run whole decode
    steps (selection + attention of one query row) until `seconds` elapse."""
    import numpy as np
    import oracle
    ncores = max(1, min(16, len(os.sched_getaffinity(0))))
    d = oracle.Dims(B=w.B, L=w.L, ratio=w.ratio, window=w.window, topk=w.topk, index_block=w.index_block,
                    index_keep=w.index_keep, H_i=w.H_i, D_i=w.D_i, H=w.H, Dk=w.Dk, Dv=w.Dv, Np_cap=int(x["Np_cap"]))
    oracle.lib()
    rows = [(b, j) for b in range(w.B) for j in range(w.L)]
    done = [0] * ncores
    stop_at = time.perf_counter() + seconds

    def work(tid):
        i = tid
        while time.perf_counter() < stop_at:
            b, j = rows[i % len(rows)]
            t0 = int(x["t0"][b])
            I, _, _ = oracle.select_row(d, x["q_idx"][b, j], x["w"][b, j], x["keys"][b], t0, j)
            oracle.combine_row(d, x["q"][b, j], x["local_kv"][b], x["pooled_kv"][b], I, x["sinks"], t0, j)
            done[tid] += 1
            i += ncores

    t_start = time.perf_counter()
    th = [threading.Thread(target=work, args=(t,)) for t in range(ncores)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    el = time.perf_counter() - t_start
    n = sum(done)
    return {"value": n / el, "unit": "rows/s", "cores": ncores, "kind": "oracle",
            "sample": f"{n} query rows of {w.name} (selection + attention per row, whole rows on "
                      f"{ncores} host threads for {el:.1f} s)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from top_kv_indexer_amd import hisa, synth

    if args.calibrate_copy:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(w, synth.SEEDS[w.name])
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.bf16 else torch.float32
    L = hisa.lib()

    def put(a, dtype=dt):
        return torch.from_numpy(a).to(dev).to(dtype).contiguous()

    base = {k: put(x[k]) for k in ("q_idx", "keys", "q", "local_kv", "pooled_kv")}
    base["w"] = put(x["w"], torch.float32)
    t0 = put(x["t0"], torch.int32)
    sinks = put(x["sinks"], torch.float32) if x["sinks"] is not None else None
    per_copy = sum(v.numel() * v.element_size() for v in base.values())
    R = max(2, -(-MALL_DEFEAT_BYTES // per_copy))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]

    kind = "decode" if (w.L == 1 and w.index_block) else ("prefill" if w.index_block else "flat")
    sel_d = hisa.selection_dims(base["q_idx"], base["keys"], ratio=w.ratio, topk=w.topk,
                                index_block=w.index_block, index_keep=w.index_keep)
    I = torch.empty((w.B, w.L, w.topk), dtype=torch.int32, device=dev)
    blk = torch.empty((w.B, w.L, w.index_keep), dtype=torch.int32, device=dev)
    path = torch.empty((w.B,), dtype=torch.int32, device=dev)
    att_d = hisa.attention_dims(base["q"], base["local_kv"] if w.window else None, base["pooled_kv"], I,
                                ratio=w.ratio, window=w.window)
    out = torch.empty((w.B, w.L, w.H, w.Dv), dtype=dt, device=dev)
    op = {"decode": hisa.OP_SELECT_DECODE, "prefill": hisa.OP_SELECT_PREFILL, "flat": hisa.OP_FLAT_TOPK}[kind]
    ws_sel = torch.zeros(max(hisa.workspace_bytes(op, sel_d), 256), dtype=torch.uint8, device=dev)
    ws_att = torch.zeros(max(hisa.workspace_bytes(hisa.OP_ATTENTION, att_d), 256), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sel_ref, att_ref = ctypes.byref(sel_d), ctypes.byref(att_d)
    n_sel, n_att = ws_sel.numel(), ws_att.numel()

    # Pre-bound C calls (argument marshalling done once per copy).
    calls = []
    for c in copies:
        if kind == "flat":
            a_sel = (sel_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(t0), P(I), P(ws_sel), n_sel, stream)
            f_sel = L.flat_topk_select
        else:
            a_sel = (sel_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(t0), P(I), P(blk), P(path), P(ws_sel),
                     n_sel, stream)
            f_sel = L.hisa_select_decode if kind == "decode" else L.hisa_select_prefill
        a_att = (att_ref, P(c["q"]), P(c["local_kv"]) if w.window else None, P(c["pooled_kv"]), P(I), P(sinks),
                 P(t0), P(out), P(ws_att), n_att, stream)
        calls.append((f_sel, a_sel, L.sparse_local_pooled_attention, a_att))

    def step(i):
        f1, a1, f2, a2 = calls[i % R]
        rc = f1(*a1)
        rc |= f2(*a2)
        if rc:
            raise hisa.HisaError(hisa.last_error())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            # the library launches on the stream it is given: point it at the capture stream
            cap = ctypes.c_void_p(s.cuda_stream)
            for i in range(args.steps):
                f1, a1, f2, a2 = calls[i % R]
                f1(*a1[:-1], cap)
                f2(*a2[:-1], cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    # Timed region: K steps back to back.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps

    # Same steps again with the library's per-kernel HIP events (kernel roofline).
    hisa.hisa_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = hisa.hisa_profile_collect()
    hisa.hisa_profile_enable(False)

    In = I.cpu().numpy()
    uniq = 0
    for b in range(w.B):
        ids = In[b].reshape(-1)
        uniq += len(np.unique(ids[(ids >= 0) & (ids < int(x["Np"][b]))]))
        uniq += int(x["Wl"][b]) if w.window else 0
    # flat_topk_select has no path output: every sequence is on the flat path
    flat_seqs = [True] * w.B if kind == "flat" else [int(v) == hisa.PATH_FLAT for v in path.cpu().tolist()]
    alg = algorithmic(w, x, unique_kv_rows=uniq, flat_seqs=flat_seqs)
    kernels = {}
    for name, (n, tot) in prof.items():
        avg_ms = tot / max(n, 1)
        kernels[name] = {"launches_per_step": n // args.steps, "avg_us": round(avg_ms * 1e3, 3)}
        if name in alg and avg_ms > 0:
            kernels[name].update(rate(alg[name], avg_ms / 1e3))
    dominant = max(prof.items(), key=lambda kv: kv[1][1])[0]
    dom_avg_s = prof[dominant][1] / prof[dominant][0] / 1e3
    timing = "HIP events around each launch"
    # A per-launch event pair adds a few microseconds, which matters for
    # microsecond kernels: when the library call holding the dominant kernel
    # launches that kernel alone, time K back-to-back calls between two
    # events on the library stream instead.
    sel_kernels = {"decode": ("decode_scan_select",), "prefill": (), "flat": ()}[kind]
    alone = None
    if dominant in sel_kernels and set(prof) & {"decode_scan", "decode_select"} == set():
        alone = 0
    elif dominant == "attention" and "attention_merge" not in prof:
        alone = 2
    if alone is not None:
        torch.cuda.synchronize()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(args.steps):
            f, a_ = calls[i % R][alone], calls[i % R][alone + 1]
            if f(*a_):
                raise hisa.HisaError(hisa.last_error())
        e3.record()
        torch.cuda.synchronize()
        dom_avg_s = e2.elapsed_time(e3) / args.steps / 1e3
        timing = f"{args.steps} back-to-back launches of its library call between two HIP events"
    a = alg.get(dominant, {"bytes": 0, "flops": 0})
    roof = rate(a, dom_avg_s)
    roof["peak"] = BF16_PEAK_TFLOPS if roof["bound"] == "mfma" else HBM_PEAK_GBPS
    roof["traffic"] = stored_traffic(w.name, dominant)
    roof["kernel"] = dominant
    roof["algorithmic_per_launch"] = a["flops"] if roof["bound"] == "mfma" else a["bytes"]
    roof["avg_us"] = round(dom_avg_s * 1e6, 3)
    roof["timing"] = timing

    step_bytes = sum(alg[k]["bytes"] for k in prof if k in alg and k not in ("attention_merge", "decode_select",
                                                                                "topk_rows"))
    rows = w.B * w.L
    res = {
        "metric": METRIC,
        "value": round(rows / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "Np": [int(n) for n in x["Np"]][:4],
                   "H_i": w.H_i, "D_i": w.D_i, "topk": w.topk, "index_block": w.index_block,
                   "index_keep": w.index_keep, "H": w.H, "head_dim": w.Dk, "window": w.window,
                   "us_per_layer": round(ms * 1e3, 3), "step_algorithmic_bytes": step_bytes,
                   "step_GBps": round(step_bytes / (ms / 1e3) / 1e9, 1), "input_copies_cycled": R,
                   "hip_graph": bool(args.graph), "wall_s": round(wall, 4)},
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
