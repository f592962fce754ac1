#!/usr/bin/env python3
"""Benchmark of the HiSA hot path on one MI355X.

A step is one layer's pass of the whole path over one batch of synthetic
input: selection (gate, block means, coarse top-Kb, fine top-k, or the flat
scan) followed by the sparse local + pooled attention that consumes it.  The
default workload is one V4-Flash-shaped decode step at Np = 16384 pooled keys
(B = 1, 64 x 128 bf16 indexer, top-512 of blocks of 64, 64 heads x 512, window
128, sinks).  Inputs are resident in HBM before timing starts.

Timing (HIP events on the stream the library launches on, created with
hipEventDisableSystemFence: a default event's record adds a system-scope
cache writeback and invalidation, ~3 us, to the interval it closes; these
events time the launches between them, as the profiler's kernel trace does):
  cold  before every step a kernel reads a 1 GiB buffer (outside the step's
        events), which evicts the step's data from the 256 MiB Infinity Cache
        and the L2s; K steps, each between its own pair of events; the median
        is the headline, p10 / p90 beside it;
  hot   K steps back to back between two events (data partly cache resident);
  graph one step captured into a HIP graph and replayed, cold and hot.
Selection alone is timed cold the same way.

Prints ONE JSON line: rows/s (B*L / cold median step time), us per layer,
step GB/s, the roofline of the dominant kernel (its algorithmic bytes or
flops per launch over its cold median duration, from HIP events around its
library call when that call launches it alone), and the CPU oracle timed on
the host's cores on a bounded sample of the same workload.
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
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="v4flash_decode_np16384")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay figures")
    ap.add_argument("--selector", choices=("auto", "cached", "stateless"), default="auto",
                    help="decode selection: re-reading every key (the faster at B = 1 below Np ~ 100K) or on "
                         "cached block means (the step keeps the cache current; flat in Np, faster for batches); "
                         "auto takes the cached means for batches of 8+ rows or Np >= 131072, as measured")
    ap.add_argument("--step-call", choices=("decode_step", "two_calls"), default="decode_step",
                    help="decode with the stateless selector: hisa_decode_step (selection and attention in one call, "
                         "one kernel for few sequences) or hisa_select_decode then sparse_local_pooled_attention")
    ap.add_argument("--crossover", action="store_true",
                    help="flat vs HiSA decode selection and sparse vs dense prefill attention against Np")
    ap.add_argument("--sweep-np", action="store_true",
                    help="decode step time against the pooled count (both selectors), one JSON line per Np")
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
        # selection and attention in one kernel: the step's whole compulsory traffic
        "decode_step": {"bytes": keys + idx_q + rows * kI * 4 + attn_bytes,
                        "flops": sum(Np) * w.H_i * w.D_i * 2 + attn_flops},
        "attention": {"bytes": attn_bytes, "flops": attn_flops},
        "attention_merge": {"bytes": rows * w.H * w.Dv * bf, "flops": 0},
        "block_mean": {"bytes": keys, "flops": 0},
        "coarse": {"bytes": idx_q, "flops": L * sum(nb) * w.H_i * w.D_i * 2},
        "fine": {"bytes": idx_q + rows * kI * 4, "flops": rows * C * w.H_i * w.D_i * 2},
        # the flat scan scores only the sequences on the flat path
        "flat_scores": {"bytes": sum(Np[b] for b in flat) * w.D_i * bf + len(flat) * L * (w.H_i * w.D_i * bf + w.H_i * 4),
                        "flops": sum(sum(min(Np[b], (int(x["t0"][b]) + j + 1) // w.ratio) for j in range(L))
                                     for b in flat) * w.H_i * w.D_i * 2},
        # the row top-k reads each flat row's scores (an intermediate of the
        # step, but this kernel's input) and writes its ids
        "topk_rows": {"bytes": sum(Np[b] for b in flat) * L * 4 + len(flat) * L * kI * 4, "flops": 0},
        # the cached decode reads each sequence's block means and its C candidate rows
        "cached_decode": {"bytes": sum(nbb * w.D_i * 4 + min(C, n) * w.D_i * bf for nbb, n in zip(nb, Np))
                          + idx_q + rows * kI * 4,
                          "flops": sum(nb) * w.H_i * w.D_i * 2 + sum(min(C, n) for n in Np) * w.H_i * w.D_i * 2},
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, seconds):
    """The oracle (as it stands) on the host: threads each run whole query
    rows (selection + attention of one row) until `seconds` elapse.  Threads:
    OMP_NUM_THREADS when set (the host's CPU share), else every core in this
    process's affinity set."""
    import oracle
    affinity = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    ncores = max(1, int(env)) if env.isdigit() else affinity
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
                      f"{ncores} host threads for {el:.1f} s)",
            "cpu_model": cpu_model(), "affinity_cores": affinity,
            "threads_from": "OMP_NUM_THREADS" if env.isdigit() else "sched_getaffinity"}


class HipEvent:
    """A timing event of the HIP runtime that torch and the library share,
    recorded on torch's current stream (the stream the library launches on)
    without the system-scope fence of a default event."""
    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            import torch  # noqa: F401  (loads the runtime; the soname below then names that copy)
            h = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.e = ctypes.c_void_p()
        r = self._rt().hipEventCreateWithFlags(ctypes.byref(self.e), self._DISABLE_SYSTEM_FENCE)
        if r:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({r})")

    def record(self):
        import torch
        r = self._rt().hipEventRecord(self.e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if r:
            raise RuntimeError(f"hipEventRecord failed ({r})")

    def elapsed_time(self, end):
        """Milliseconds from this event to end (both complete)."""
        ms = ctypes.c_float()
        r = self._rt().hipEventElapsedTime(ctypes.byref(ms), self.e, end.e)
        if r:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return ms.value

    def __del__(self):
        if self.e and HipEvent._hip is not None:
            HipEvent._hip.hipEventDestroy(self.e)
            self.e = ctypes.c_void_p()


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean()), "n": int(a.size)}


_flush_state = {}


def flush():
    """The cache flush: a read of 1 GiB (evicts the step's lines from the
    Infinity Cache and the L2s; dirty ones are written back during the
    flush, not during the step)."""
    import torch
    if not _flush_state:
        _flush_state["buf"] = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        _flush_state["out"] = torch.empty((), dtype=torch.float32, device="cuda:0")
    torch.sum(_flush_state["buf"], dim=0, out=_flush_state["out"])


def harness(w, x, selector, step_call="two_calls"):
    """Device copies of workload w's inputs x, outputs and workspaces, and the
    step's C calls with their arguments marshalled once (stateless decode
    with step_call "decode_step": the one call that selects and attends)."""
    from types import SimpleNamespace

    import torch
    from top_kv_indexer_amd import hisa
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.bf16 else torch.float32
    L = hisa.lib()

    def put(a, dtype=dt):
        return torch.from_numpy(a).to(dev).to(dtype).contiguous()

    base = {k: put(x[k]) for k in ("q_idx", "keys", "q", "local_kv", "pooled_kv")}
    base["w"] = put(x["w"], torch.float32)
    t0 = put(x["t0"], torch.int32)
    sinks = put(x["sinks"], torch.float32) if x["sinks"] is not None else None
    kind = "decode" if (w.L == 1 and w.index_block) else ("prefill" if w.index_block else "flat")
    sel_d = hisa.selection_dims(base["q_idx"], base["keys"], ratio=w.ratio, topk=w.topk,
                                index_block=w.index_block, index_keep=w.index_keep)
    I = torch.empty((w.B, w.L, w.topk), dtype=torch.int32, device=dev)
    blk = torch.empty((w.B, w.L, w.index_keep), dtype=torch.int32, device=dev)
    path = torch.empty((w.B,), dtype=torch.int32, device=dev)
    att_d = hisa.attention_dims(base["q"], base["local_kv"] if w.window else None, base["pooled_kv"], I,
                                ratio=w.ratio, window=w.window)
    out = torch.empty((w.B, w.L, w.H, w.Dv), dtype=dt, device=dev)
    cached = kind == "decode" and selector == "cached"
    op = {"decode": hisa.OP_SELECT_DECODE_CACHED if cached else hisa.OP_SELECT_DECODE,
          "prefill": hisa.OP_SELECT_PREFILL, "flat": hisa.OP_FLAT_TOPK}[kind]
    rep = None
    if cached:
        # the cache as a decode loop keeps it: every block complete before this step
        _, rep = hisa.hisa_block_scores(base["q_idx"], base["w"], base["keys"], t0, ratio=w.ratio,
                                        index_block=w.index_block, want_rep=True)
    ws_sel = torch.zeros(max(hisa.workspace_bytes(op, sel_d), 256), dtype=torch.uint8, device=dev)
    one_call = kind == "decode" and not cached and step_call == "decode_step"
    step_d = hisa.decode_step_dims(base["q_idx"], base["keys"], base["q"], base["local_kv"] if w.window else None,
                                   base["pooled_kv"], ratio=w.ratio, window=w.window, topk=w.topk,
                                   index_block=w.index_block, index_keep=w.index_keep) if one_call else None
    ws_step = torch.zeros(max(hisa.workspace_bytes(hisa.OP_DECODE_STEP, step_d), 256), dtype=torch.uint8,
                          device=dev) if one_call else None
    ws_att = torch.zeros(max(hisa.workspace_bytes(hisa.OP_ATTENTION, att_d), 256), dtype=torch.uint8, device=dev)
    main_stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sel_ref, att_ref = ctypes.byref(sel_d), ctypes.byref(att_d)
    step_ref = ctypes.byref(step_d) if one_call else None
    n_sel, n_att = ws_sel.numel(), ws_att.numel()
    c = base

    def bound_calls(stream_handle):
        """The step's two C calls with their arguments marshalled once."""
        st = ctypes.c_void_p(stream_handle)
        if kind == "flat":
            a_sel = (sel_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(t0), P(I), P(ws_sel), n_sel, st)
            f_sel = L.flat_topk_select
        elif cached:
            a_sel = (sel_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(rep), P(t0), P(I), P(blk), P(path),
                     P(ws_sel), n_sel, st)
            f_sel = L.hisa_select_decode_cached
        else:
            a_sel = (sel_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(t0), P(I), P(blk), P(path), P(ws_sel),
                     n_sel, st)
            f_sel = L.hisa_select_decode if kind == "decode" else L.hisa_select_prefill
        a_att = (att_ref, P(c["q"]), P(c["local_kv"]) if w.window else None, P(c["pooled_kv"]), P(I), P(sinks),
                 P(t0), P(out), P(ws_att), n_att, st)
        a_step = (step_ref, P(c["q_idx"]), P(c["w"]), P(c["keys"]), P(c["q"]), P(c["local_kv"]) if w.window else None,
                  P(c["pooled_kv"]), P(sinks), P(t0), P(I), P(blk), P(path), P(out), P(ws_step),
                  ws_step.numel(), st) if one_call else None
        return f_sel, a_sel, L.sparse_local_pooled_attention, a_att, L.hisa_decode_step, a_step

    f1, a1, f2, a2, f3, a3 = bound_calls(main_stream.cuda_stream)

    def call(f, a):
        if f(*a):
            raise hisa.HisaError(hisa.last_error())

    def step(i=0):
        if one_call:
            call(f3, a3)
            return
        call(f1, a1)
        call(f2, a2)

    def sel_only(i=0):
        call(f1, a1)

    def att_only(i=0):
        call(f2, a2)

    def cold(fn, k):
        """k runs of fn, each after a flush and between its own two events;
        returns the per-run milliseconds."""
        ev = [(HipEvent(), HipEvent()) for _ in range(k)]
        for i in range(k):
            flush()
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def hot(fn, k):
        e0, e1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        e0.record()
        for i in range(k):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    return SimpleNamespace(**{k: v for k, v in locals().items() if k not in ("h", "SimpleNamespace")})


def cold_ms(fn, k):
    """k runs of fn(i), each after a flush and between its own two HIP events
    (on the current stream); the median milliseconds."""
    import torch
    ev = [(HipEvent(), HipEvent()) for _ in range(k)]
    for i in range(k):
        flush()
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return percentiles([a.elapsed_time(b) for a, b in ev])["median"]


def crossover(args):
    """The pages' engagement thresholds re-measured here (cold medians, one
    JSON line per point): (1) decode selection, flat scan vs HiSA (re-reading
    the keys, and on cached block means) at B = 1 for Np around the 1024
    threshold; (2) a 512-row prefill chunk, selection + sparse attention vs
    dense attention over every visible pooled row, against Np."""
    import torch
    from top_kv_indexer_amd import hisa, synth
    dev = torch.device("cuda:0")
    bf = torch.bfloat16

    def put(a, dt=bf):
        return torch.from_numpy(a).to(dev).to(dt).contiguous()

    for Np in (600, 800, 1000, 1024, 1536, 2048, 4096, 8192, 16384, 32768):
        w = synth.FLASH_DECODE.with_(name=f"crossover_decode_np{Np}", t0=[4 * Np], Np_cap=Np,
                                     planted=min(32, Np // 64))
        x = synth.make_inputs(w, 77, need_attention=False)
        q, wt, keys, t0 = put(x["q_idx"]), put(x["w"], torch.float32), put(x["keys"]), put(x["t0"], torch.int32)
        I = torch.empty((1, 1, 512), dtype=torch.int32, device=dev)
        blk = torch.empty((1, 1, 16), dtype=torch.int32, device=dev)
        path = torch.empty((1,), dtype=torch.int32, device=dev)
        kw = dict(ratio=4, topk=512, index_block=64, index_keep=16, I=I, top_blk=blk, path=path)
        line = {"kind": "decode_selection", "Np": Np}
        hisa.hisa_select_decode(q, wt, keys, t0, **kw)
        torch.cuda.synchronize()
        line["gate"] = {0: "dense", 1: "flat", 2: "hisa"}[int(path[0])]
        line["flat_us"] = round(1e3 * cold_ms(lambda i: hisa.hisa_select_decode(q, wt, keys, t0, mode=1, **kw),
                                              args.steps), 3)
        if line["gate"] == "hisa":
            line["hisa_us"] = round(1e3 * cold_ms(lambda i: hisa.hisa_select_decode(q, wt, keys, t0, **kw),
                                                  args.steps), 3)
            _, rep = hisa.hisa_block_scores(q, wt, keys, t0, ratio=4, index_block=64, want_rep=True)
            line["hisa_cached_us"] = round(1e3 * cold_ms(
                lambda i: hisa.hisa_select_decode_cached(q, wt, keys, rep, t0, **kw), args.steps), 3)
        print(json.dumps(line), flush=True)
    L = 512
    for Np in (512, 1024, 2048, 4096, 8192, 16384):
        w = synth.PREFILL.with_(name=f"crossover_prefill_np{Np}", L=L, t0=[4 * Np - L])
        x = synth.make_inputs(w, 78)
        g = {k: put(x[k]) for k in ("q_idx", "keys", "q", "local_kv", "pooled_kv")}
        wt, t0, sinks = put(x["w"], torch.float32), put(x["t0"], torch.int32), put(x["sinks"], torch.float32)
        I = torch.empty((1, L, 512), dtype=torch.int32, device=dev)
        out = torch.empty((1, L, 64, 512), dtype=bf, device=dev)
        line = {"kind": "prefill_chunk_l512", "Np": Np}

        def sparse(i):
            hisa.hisa_select_prefill(g["q_idx"], wt, g["keys"], t0, ratio=4, topk=512, index_block=64, index_keep=16,
                                     I=I)
            hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], I, sinks, t0, ratio=4,
                                               window=128, out=out)

        def dense(i):
            hisa.sparse_local_pooled_attention(g["q"], g["local_kv"], g["pooled_kv"], None, sinks, t0, ratio=4,
                                               window=128, out=out)

        line["sparse_us"] = round(1e3 * cold_ms(sparse, max(3, args.steps // 4)), 3)
        line["dense_us"] = round(1e3 * cold_ms(dense, max(3, args.steps // 4)), 3)
        print(json.dumps(line), flush=True)
        del g


def sweep_np(args):
    """Cold decode times against the pooled count, for both selectors: one
    JSON line per Np (B = 1, the V4-Flash shapes otherwise)."""
    import torch  # noqa: F401
    from top_kv_indexer_amd import synth
    for Np in (4096, 8192, 16384, 32768, 65536, 131072, 262144):
        w = synth.FLASH_DECODE.with_(name=f"v4flash_decode_np{Np}", t0=[4 * Np], Np_cap=Np)
        x = synth.make_inputs(w, synth.SEEDS[synth.FLASH_DECODE.name])
        line = {"Np": Np}
        for sel in ("stateless", "cached"):
            H = harness(w, x, sel, args.step_call)
            for i in range(args.warmup):
                flush()
                H.step(i)
            line[sel] = {"selection_cold_us": round(percentiles(H.cold(H.sel_only, args.steps))["median"] * 1e3, 3),
                         "step_cold_us": round(percentiles(H.cold(H.step, args.steps))["median"] * 1e3, 3),
                         "step_hot_us": round(H.hot(H.step, args.steps) * 1e3, 3)}
            del H
        print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
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
    if args.sweep_np:
        return sweep_np(args)
    if args.crossover:
        return crossover(args)
    selector = args.selector
    if selector == "auto":
        selector = "cached" if (w.B * w.L >= 8 or int(max(x["Np"])) >= 131072) else "stateless"
    H = harness(w, x, selector, args.step_call)
    dev, I, blk, path, kind, cached, one_call = H.dev, H.I, H.blk, H.path, H.kind, H.cached, H.one_call
    step, sel_only, att_only, cold, hot, call, bound_calls = (H.step, H.sel_only, H.att_only, H.cold, H.hot, H.call,
                                                             H.bound_calls)
    main_stream = H.main_stream

    for i in range(args.warmup):
        flush()
        step(i)
    torch.cuda.synchronize()

    # Timed region: K cold steps (a flush before each, outside its events).
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_ms = cold(step, args.steps)
    wall = time.perf_counter() - wall0
    cold_step = percentiles(step_ms)
    ms = cold_step["median"]
    hot_ms = hot(step, args.steps)
    sel_cold = percentiles(cold(sel_only, args.steps))

    graph_fig = None
    if not args.no_graph:
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(main_stream)
        graph = torch.cuda.CUDAGraph()
        g1, b1, g2, b2, g3, b3 = bound_calls(s.cuda_stream)
        with torch.cuda.graph(graph, stream=s):
            if one_call:
                call(g3, b3)
            else:
                call(g1, b1)
                call(g2, b2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_cold = percentiles(cold(lambda i: graph.replay(), args.steps))
        g_hot = hot(lambda i: graph.replay(), args.steps)
        graph_fig = {"cold_median_us": round(g_cold["median"] * 1e3, 3), "cold_p10_us": round(g_cold["p10"] * 1e3, 3),
                     "cold_p90_us": round(g_cold["p90"] * 1e3, 3), "hot_us": round(g_hot * 1e3, 3)}

    # Kernel ranking: the same cold steps with the library's per-kernel HIP
    # events (each launch between its own two events).
    hisa.hisa_profile_enable(True)
    for i in range(args.steps):
        flush()
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
    prof = {k: v for k, v in prof.items() if v[0] > 0}
    dominant = max(prof.items(), key=lambda kv: kv[1][1])[0]
    dom_avg_s = prof[dominant][1] / prof[dominant][0] / 1e3
    timing = "cold; mean of per-launch HIP event pairs (library kernel timing)"
    # When the library call holding the dominant kernel launches that kernel
    # alone, time that call: cold, its own event pair per launch, median.
    sel_kernels = {"decode": ("decode_scan_select",), "prefill": (), "flat": ()}[kind]
    alone = None
    if dominant in sel_kernels and set(prof) & {"decode_scan", "decode_select"} == set():
        alone = sel_only
    elif dominant == "attention" and "attention_merge" not in prof:
        alone = att_only
    if alone is not None:
        dom = percentiles(cold(alone, args.steps))
        dom_avg_s = dom["median"] / 1e3
        timing = f"cold; median of {args.steps} launches of its library call, each between two HIP events"
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
    us = lambda v: round(v * 1e3, 3)  # noqa: E731
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
                   "selector": ("cached block means" if cached else "every key re-read") if kind == "decode"
                   else kind,
                   "step_call": "hisa_decode_step" if one_call else "selection call + attention call",
                   "us_per_layer": us(ms), "step_algorithmic_bytes": step_bytes,
                   "step_GBps": round(step_bytes / (ms / 1e3) / 1e9, 1),
                   "timing": "cold: 1 GiB read flush before each step, outside its HIP events; median",
                   "cold_step_us": {"median": us(ms), "p10": us(cold_step["p10"]), "p90": us(cold_step["p90"])},
                   "hot_step_us": us(hot_ms),
                   "selection_only": {"rows_per_s": round(rows / (sel_cold["median"] / 1e3), 1),
                                      "cold_median_us": us(sel_cold["median"]), "cold_p10_us": us(sel_cold["p10"]),
                                      "cold_p90_us": us(sel_cold["p90"])},
                   "hip_graph_step": graph_fig, "wall_s": round(wall, 4),
                   "kernels_timing": "cold steps; per launch, the mean of its own HIP event pair (event cost included)"},
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
