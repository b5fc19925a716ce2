"""Benchmark of the WeDLM streaming window step on one MI355X.

Default workload: the Qwen3-8B-shaped streaming loop - 36 independent layers'
paged KV caches, 16 sequences, initial prefix 1024, window 16, vocabulary
151936, bf16 - run for --steps window steps (256 by default: the whole loop)
after --warmup steps from the same start state. Every timed step is the whole
path: reorder, window attention over all 36 layers with RoPE at the logical
positions applied as the window is loaded (the same call appends the committed
rows to the cache), entropy/selection over the full vocabulary, and the
commit of the window state (shift and refill). Inputs are
synthetic and already resident in HBM when timing starts.

Prints one JSON line: window-steps/s (value), committed tokens/s, the HBM rate
of the algorithmic bytes (KV prefix + window + logits + committed rows) per
step, the roofline of the dominant kernel (window attention, which in the
fused step also appends the committed rows) timed with HIP events on the
launch stream, and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
# counted HBM bytes of the attention launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
# calibrated); used only while the kernel source still matches the record
TRAFFIC_RECORD = "k_window_attn_bf16_qwen3_36L_bs16_stream256_traffic.txt"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen3_8b_36L_bs16_L1024_W16_stream256")
    ap.add_argument("--cpu-baseline-steps", type=int, default=2,
                    help="window steps of the oracle timed on the host (0 disables; one step of "
                         "the streaming workload is ~8 s of fp64 work on 16 host cores)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead: single-step latency of every other workload, one JSON line each")
    ap.add_argument("--lm-head", action="store_true",
                    help="time the fused vocabulary projection + selection (one JSON line per shape)")
    ap.add_argument("--lm-head-steps", type=int, default=50)
    ap.add_argument("--decode-modes", action="store_true",
                    help="streaming vs one-by-one vs block-wise decoding on the same kernels "
                         "(one JSON line per mode and logit regime)")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--dual-stream", action="store_true",
                    help="time the dual-stream masking attention forward (one JSON line per block size)")
    ap.add_argument("--read-bw", action="store_true",
                    help="HBM read-rate probe (plain streaming read and random 4 KB blocks, the "
                         "paged cache's pattern) as context for the roofline fractions")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record the attention / entropy timing events on every n-th timed "
                         "step (each record idles the GPU for a few microseconds)")
    ap.add_argument("--separate-entropy", action="store_true",
                    help="run each step's entropy chunk pass as its own launch after the "
                         "attention (by default it rides in the attention's launch)")
    ap.add_argument("--overlap", action="store_true",
                    help="run each step's entropy chunk pass on a second stream beside the "
                         "attention (fused tail only)")
    ap.add_argument("--separate-tail", action="store_true",
                    help="chained steps run selection, state commit and reorder as three calls "
                         "instead of the fused tail")
    ap.add_argument("--config-steps", type=int, default=200)
    ap.add_argument("--config-warmup", type=int, default=20)
    ap.add_argument("--only", default=None,
                    help="with --all-configs: time only this workload (e.g. to trace it alone)")
    ap.add_argument("--reps", type=int, default=3,
                    help="timed repetitions of the --steps steps, each from the same start "
                         "state (restored from a snapshot between them); the median is reported")
    return ap.parse_args()


class HipEvents:
    """Timing-only HIP events recorded on the launch stream.

    Created with hipEventDisableSystemFence: recording them does not write
    back and invalidate the caches, which a default timing event does and
    which costs about 5 us of GPU time per record between kernels. The HIP
    runtime is the one torch has already loaded (same soname).
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream_handle=0):
        import ctypes
        self.c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream_handle)
        self.events = []

    def create(self):
        e = self.c.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.c.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(e)
        return e

    def record(self, e):
        rc = self.hip.hipEventRecord(e, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        rc = self.hip.hipEventElapsedTime(self.c.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def step_bytes(wl, prefix_lens, commits):
    """Algorithmic HBM bytes of one window step, split by tensor (each byte once).

    commits: rows committed per sequence this step (their K and V rows are
    written to the cache, by the attention call in the fused step).
    """
    e = 2 if wl.dtype == "bf16" else 4
    kv = int(sum(prefix_lens)) * wl.n_layers * wl.Hkv * wl.D * 2 * e
    win_in = wl.n_layers * wl.B * wl.W * (wl.Hq + 2 * wl.Hkv) * wl.D * e
    attn_out = wl.n_layers * wl.B * wl.W * wl.Hq * wl.D * e
    commit = int(sum(commits)) * wl.n_layers * wl.Hkv * wl.D * 2 * e
    logits = wl.B * wl.W * wl.V * e
    return {"kv": kv, "window": win_in, "attn_out": attn_out, "commit": commit, "logits": logits}


def cpu_baseline(wl, inp, host_steps):
    """The oracle (never tuned) on the first steps of the same workload, on the host."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = 1
    cores = len(os.sched_getaffinity(0))
    kc = [[np.asarray(x, np.float64) for x in inp["k_cache"][l]] for l in range(wl.n_layers)]
    vc = [[np.asarray(x, np.float64) for x in inp["v_cache"][l]] for l in range(wl.n_layers)]
    t0 = time.perf_counter()
    out = oracle.stream_loop(inp["filled"], inp["tokens"], inp["prefix_len"], kc, vc,
                             inp["block_table"], len(host_steps), lambda s: host_steps[s], wl.theta,
                             wl.lam, wl.tau, wl.page_size, wl.min_fill, wl.mask_id,
                             attend=lambda s: range(wl.n_layers), track_layers=range(wl.n_layers))
    dt = time.perf_counter() - t0
    n = len(host_steps)
    return {"value": n / dt, "unit": "window-steps/s", "cores": max(threads, 1),
            "host_cpus": cores, "kind": "oracle",
            "sample": f"first {n} window steps of the same workload, all {wl.n_layers} layers and "
                      f"{wl.B} sequences (fp64 NumPy oracle, {dt:.1f} s, "
                      f"{out['total_committed']} tokens committed)"}


def entropy_report(entropy, filled, score, tau):
    """Histogram of the slot entropies (nats, unit bins) and how often the
    threshold fires among mask slots: the logits' regime, from the kernels'
    own output."""
    import numpy as np

    H = np.asarray(entropy, np.float64).ravel()
    mask = ~np.asarray(filled, bool).ravel()
    sc = np.asarray(score, np.float64).ravel()
    top = int(np.ceil(max(float(H.max()), 1.0)))
    counts, edges = np.histogram(H, bins=np.arange(0, top + 1))
    return {"unit": "nats", "bins": [f"[{int(a)},{int(b)})" for a, b in zip(edges[:-1], edges[1:])],
            "counts": counts.tolist(), "slots": int(H.size), "min": float(H.min()),
            "median": float(np.median(H)), "max": float(H.max()),
            "mask_slots": int(mask.sum()),
            "mask_slots_below_tau": int((sc[mask] < tau).sum())}


def config_latencies(args):
    """Single-step latency of each single-step workload (one JSON line each).

    Every timed step starts from the same state (restored outside the timed
    pair) and follows a 512 MB read that evicts the caches' contents, so the
    KV prefix and logits come from HBM as in a real decoder. The step is the
    streaming loop's launch sequence (reorder, attention with fused RoPE and
    append, split combine where split, entropy pass, fused tail), captured
    once as a HIP graph and replayed between two timing events: nothing else
    sits between the step's kernels (for bf16 the entropy chunk pass rides in
    the attention's launch). Reported: the median, p10 and p90 of the
    replayed step; the same step launched eagerly (one host call per kernel);
    eagerly with the entropy chunk pass as a launch of its own after the
    attention, and on a second stream beside it (it reads only the logits);
    and, from an eager pass with timing events between the kernels, the
    attention and entropy + tail segments (each event record adds a few
    microseconds of idle GPU, so these are upper bounds of the kernels; the
    kernel trace gives their own durations). HBM rates use the algorithmic
    bytes over the segment medians. The slot entropies of the step are
    reported as a histogram.
    """
    import numpy as np
    import torch

    from causal_streaming_decoding_amd import workloads as WL
    from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
    from causal_streaming_decoding_amd.synth import make_step_inputs

    dev = "cuda:0"
    # evicting by reading leaves no dirty lines whose write-back would land
    # inside the next timed step (a 512 MB write would leave up to the whole
    # 256 MB infinity cache dirty)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MB
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)
    hev = HipEvents(torch.cuda.current_stream().cuda_stream)
    labels = ("step_start", "attn_start", "attn_end", "entropy_end", "step_end")
    n = args.config_warmup + args.config_steps
    for wl in WL.ALL:
        if wl.steps > 1:
            continue  # the streaming loop is the default bench line
        if args.only is not None and wl.name != args.only:
            continue
        print(f"[bench] {wl.name}", file=sys.stderr, flush=True)
        inp = make_step_inputs(wl)
        st, q, k, v, logits, mpl = upload_step_inputs(wl, inp, dev)
        # the launch sequence of the streaming loop: the selection, state commit
        # and next reorder run as one tail call after the entropy pass
        step = make_window_step(wl, inp, dev, mpl, fused_tail=True)
        snap = st.snapshot()
        graph = step.capture(st, q, k, v, logits)

        def timed(launch, marks, prep=None):
            ev = [{lab: hev.create() for lab in labels} for _ in range(n)]
            for i in range(n):
                st.restore(snap)
                if prep is not None:
                    prep()
                torch.sum(flush, dim=0, out=flush_sink)
                e = ev[i]
                hev.record(e["step_start"])
                launch((lambda lab, e=e: hev.record(e[lab])) if marks else None)
                hev.record(e["step_end"])
            torch.cuda.synchronize()
            out = {}
            spans = {"step": ("step_start", "step_end")}
            if marks:
                spans.update(attn=("attn_start", "attn_end"), entropy=("attn_end", "entropy_end"))
            for name, (a, b) in spans.items():
                out[name] = np.array([hev.elapsed_ms(x[a], x[b]) for x in ev[args.config_warmup:]]) * 1e3
            hev.destroy()
            return out

        g_span = timed(lambda mark: graph.replay(), False)
        e_span = timed(lambda mark: step.run(st, q, k, v, logits), False)
        # a step of a decoding loop: the previous step's tail already reordered
        # the window (here an untimed reorder before the cache flush)
        c_span = timed(lambda mark: step.run(st, q, k, v, logits), False,
                       prep=lambda: step.reorder(st))
        m_span = timed(lambda mark: step.run(st, q, k, v, logits, mark=mark), True)
        # the entropy chunk pass as a launch of its own after the attention
        # (bf16 runs it in the attention's launch by default) ...
        default_fuse = step.fuse_entropy
        step.fuse_entropy = False
        s_span = timed(lambda mark: step.run(st, q, k, v, logits), False)
        # ... and on a second stream beside the attention
        step.set_overlap(torch.cuda.Stream())
        o_span = timed(lambda mark: step.run(st, q, k, v, logits), False)
        step.set_overlap(None)
        step.fuse_entropy = default_fuse
        L = np.asarray(inp["prefix_len"], np.int64)
        commits = step.commit_len.cpu().numpy()
        b = step_bytes(wl, L, commits)
        attn_bytes = b["kv"] + b["window"] + b["attn_out"] + b["commit"]
        if default_fuse:
            attn_bytes += b["logits"]  # the attention launch reads the logits too
        ent = entropy_report(step.entropy.cpu().numpy(), inp["filled"], step.score.cpu().numpy(),
                             wl.tau)

        def stats(x):
            return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
                    "p90": float(np.percentile(x, 90))}

        med = {k_: float(np.median(v_)) for k_, v_ in m_span.items()}
        step_bytes_total = sum(b.values())
        line = {
            "workload": wl.name, "dtype": wl.dtype, "steps": args.config_steps,
            "warmup": args.config_warmup, "unit": "us",
            "step_us": stats(g_span["step"]), "step_launch": "one HIP graph replay",
            "entropy_pass": "in the attention's launch" if default_fuse else "own launch",
            "eager_step_us": stats(e_span["step"]),
            "chained_step_us": stats(c_span["step"]),
            "eager_separate_entropy_step_us": stats(s_span["step"]),
            "overlap_step_us": stats(o_span["step"]),
            "attn_segment_us": stats(m_span["attn"]),
            "entropy_tail_segment_us": stats(m_span["entropy"]),
            "rows": wl.B * wl.W, "vocab": wl.V,
            "step_algorithmic_bytes": int(step_bytes_total),
            "step_hbm_gbps_at_median": step_bytes_total / (float(np.median(g_span["step"])) * 1e-6) / 1e9,
            "attn_algorithmic_bytes": int(attn_bytes), "logits_bytes": int(b["logits"]),
            "attn_hbm_gbps_at_segment_median": attn_bytes / (med["attn"] * 1e-6) / 1e9,
            "entropy_hbm_gbps_at_segment_median": (None if default_fuse else
                                                   b["logits"] / (med["entropy"] * 1e-6) / 1e9),
            "entropy_histogram": ent,
            "data": "synthetic",
        }
        print(json.dumps(line), flush=True)
        del st, q, k, v, logits, step, graph
        torch.cuda.empty_cache()
    if args.calibrate_copy:
        a = torch.empty(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()


# (name, B, W, hidden, V): the projection of the streaming workload's window
# rows (Qwen3-8B), one and four sequences of it, and the Qwen2.5-7B shape
LM_HEAD_SHAPES = (
    ("qwen3_8b_lm_head_bs16_W16", 16, 16, 4096, 151936),
    ("qwen3_8b_lm_head_bs1_W16", 1, 16, 4096, 151936),
    ("qwen3_8b_lm_head_bs4_W16", 4, 16, 4096, 151936),
    ("qwen25_7b_lm_head_bs16_W32", 16, 32, 3584, 152064),
)
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, vendor figure


def lm_head_latencies(args):
    """Fused vocabulary projection + entropy selection, one JSON line per shape.

    The projection is packed once outside the timed region (model weights do
    not change between steps). Each call is timed with HIP events on the
    launch stream, back to back: the 1.2 GB projection does not fit in the
    caches, so every call streams it from HBM. Algorithmic bytes = packed
    projection + hidden states read once + outputs; flops = 2 rows hidden V.
    The roofline is HBM when the intensity (flops per byte) is below the
    bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312), else MFMA. The oracle (float64
    projection, entropy and selection) is timed on one sequence's rows.
    """
    import numpy as np
    import torch

    from causal_streaming_decoding_amd import wedlm as W
    from causal_streaming_decoding_amd.synth import lm_head_inputs, to_f64

    dev = "cuda:0"
    hev = HipEvents(torch.cuda.current_stream().cuda_stream)
    for name, B, Wn, hidden, V in LM_HEAD_SHAPES:
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        h, w, filled = lm_head_inputs(B, Wn, hidden, V, dev, seed=0)
        wp = torch.empty(W.wedlm_lm_head_packed_size(W.WEDLM_BF16, hidden, V) // 2,
                         dtype=torch.bfloat16, device=dev)
        W.wedlm_lm_head_pack(W.WEDLM_BF16, hidden, V, w, wp)
        ent = torch.empty((B, Wn), dtype=torch.float32, device=dev)
        score = torch.empty_like(ent)
        arg = torch.empty((B, Wn), dtype=torch.int32, device=dev)
        sel = torch.empty((B, Wn), dtype=torch.uint8, device=dev)
        nb = W.wedlm_lm_head_select_workspace_size(W.WEDLM_BF16, B, Wn, hidden, V)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)

        def call():
            W.wedlm_lm_head_select(W.WEDLM_BF16, B, Wn, hidden, V, h, wp, filled, 0.1, 1.0, 1, ent,
                                   score, arg, sel, ws, nb)
        n_warm, n = 5, args.lm_head_steps
        ev = [(hev.create(), hev.create()) for _ in range(n_warm + n)]
        for a_, b_ in ev:
            hev.record(a_)
            call()
            hev.record(b_)
        torch.cuda.synchronize()
        us = np.array([hev.elapsed_ms(a_, b_) for a_, b_ in ev[n_warm:]]) * 1e3
        hev.destroy()
        rows = B * Wn
        byts = wp.numel() * 2 + h.numel() * 2 + rows * (4 + 4 + 4 + 1)
        flops = 2.0 * rows * hidden * V
        med = float(np.median(us))
        intensity = flops / byts
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        if intensity < ridge:
            roof = {"bound": "hbm", "achieved": byts / (med * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": flops / (med * 1e-6) / 1e12,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = None
        # oracle on the first sequence's rows (its W rows of logits)
        import oracle
        h64 = to_f64(h[:1])
        t0 = time.perf_counter()
        z = np.concatenate([oracle.vocab_projection(h64, to_f64(w[v0:v0 + 16384]))
                            for v0 in range(0, V, 16384)], axis=-1)
        H, _ = oracle.vocab_entropy_argmax(z)
        oracle.select_slots(H[0], filled[0].cpu().numpy().astype(bool), 0.1, 1.0, 1)
        cpu_s = time.perf_counter() - t0
        line = {
            "workload": name, "metric": "vocabulary projection + selection latency", "unit": "us",
            "dtype": "bf16 (fp32 accumulation)", "rows": rows, "hidden": hidden, "V": V,
            "steps": n, "warmup": n_warm,
            "us": {"median": med, "p10": float(np.percentile(us, 10)),
                   "p90": float(np.percentile(us, 90))},
            "algorithmic_bytes": int(byts), "flops": flops, "intensity_flop_per_byte": intensity,
            "hbm_gbps_at_median": byts / (med * 1e-6) / 1e9,
            "tflops_at_median": flops / (med * 1e-6) / 1e12,
            "roofline": roof,
            "cpu_baseline": {"value": Wn / cpu_s, "unit": "rows/s", "kind": "oracle",
                             "cores": len(os.sched_getaffinity(0)),
                             "sample": f"one sequence's {Wn} rows: float64 projection, "
                                       "entropy and selection (the projection converted to "
                                       "float64 in slices, included)"},
            "data": "synthetic",
        }
        print(json.dumps(line), flush=True)
        del h, w, wp, ws
        torch.cuda.empty_cache()
    if args.calibrate_copy:
        a = torch.empty(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()


def decode_modes(args):
    """Streaming, one-by-one and block-wise decoding of the streaming workload.

    Modes (all on the same kernels, from the same start state and inputs):
    streaming (the workload's threshold, leading-run commits), one-by-one
    (threshold -inf: the single lowest-score mask per step, leading-run
    commits) and block-wise stop-and-wait (the workload's threshold, the
    window is committed only once entirely filled). Two logit regimes: the
    workload's own logits, and a low-entropy variant (spike probability 0.9,
    magnitude U[16, 20]) where the threshold fills several slots per step.
    Each mode is timed over --decode-steps window steps (steps/s, committed
    tokens/s), then replayed untimed from the same start to read its decoding
    counters (tokens and predictions per forward, p_cache, commit delay).
    """
    import dataclasses

    import numpy as np
    import torch

    from causal_streaming_decoding_amd import wedlm as Wd
    from causal_streaming_decoding_amd import workloads as WL
    from causal_streaming_decoding_amd.decode_stats import decode_counters
    from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
    from causal_streaming_decoding_amd.synth import make_step_inputs, stream_step_inputs

    dev = "cuda:0"
    K = args.decode_steps
    base = WL.BY_NAME[args.workload]
    regimes = (("workload_logits", base),
               ("low_entropy_logits", dataclasses.replace(base, spike=("prob", 0.9, 16.0, 20.0))))
    modes = (("streaming", Wd.COMMIT_STREAM, None), ("one_by_one", Wd.COMMIT_STREAM, float("-inf")),
             ("block_wise", Wd.COMMIT_BLOCK, None))
    for regime, wl0 in regimes:
        print(f"[bench] {regime}: building inputs ({K} steps)", file=sys.stderr, flush=True)
        inp = make_step_inputs(wl0, steps=K)
        ins = [stream_step_inputs(wl0, s, dev) for s in range(K)]
        for mode, rule, tau in modes:
            wl = wl0 if tau is None else dataclasses.replace(wl0, tau=tau)
            st, _, _, _, _, L0 = upload_step_inputs(wl, inp, dev)
            step = make_window_step(wl, inp, dev, L0 + wl.W * K, commit_rule=rule,
                                    fused_tail=not args.separate_tail)
            commit_log = torch.zeros((K, wl.B), dtype=torch.int32, device=dev)
            snap = st.snapshot()
            for s in range(min(8, K)):  # warm-up
                q, k, v, logits = ins[s]
                step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s)
            torch.cuda.synchronize()
            st.restore(snap)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(K):
                q, k, v, logits = ins[s]
                step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s,
                         commit_len=commit_log[s])
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
            committed = int(commit_log.sum().item())
            # untimed replay from the same start: per-step records for the counters
            st.restore(snap)
            recs = []
            for s in range(K):
                q, k, v, logits = ins[s]
                L_in = st.prefix_len.cpu().numpy()
                step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s)
                recs.append({"prefix_len_in": L_in,
                             "selected": step.selected.cpu().numpy().astype(bool),
                             "commit_len": step.commit_len.cpu().numpy()})
            c = decode_counters(recs, wl.W)
            assert c["committed"] == committed  # the replay took the timed run's path
            line = {
                "workload": base.name, "mode": mode, "logits": regime, "steps": K,
                "tau": wl.tau, "lambda": wl.lam,
                "window_steps_per_s": K / elapsed, "ms_per_step": elapsed / K * 1e3,
                "committed_tokens_per_s": committed / elapsed,
                "tokens_per_forward": c["tokens_per_forward"],
                "predictions_per_forward": c["predictions_per_forward"],
                "p_cache": c["p_cache"], "mean_commit_delay": c["mean_commit_delay"],
                "delay_histogram": {str(k_): v_ for k_, v_ in c["delay_histogram"].items()},
                "data": "synthetic",
            }
            print(json.dumps(line), flush=True)
            del st, step, commit_log
            torch.cuda.empty_cache()
        del ins
        torch.cuda.empty_cache()


def dual_stream_latencies(args):
    """Dual-stream masking attention forward of one layer, one JSON line per
    attention kernel (the block kernel, then the window kernel) and block
    size: 4 samples x 4096 positions, Qwen3-8B heads (32 / 8, D = 128),
    bf16, half of the prediction stream observed. Timed with HIP events around
    the whole forward (memory rows into the cache, both attentions, both
    reorders), 20 calls after 3 warm-up calls. Algorithmic bytes: both
    streams' q / k / v read and outputs written once, the memory rows written
    to the cache and read back once (every block re-reads its prefix, but a
    sample's memory rows - 16 MB - stay in the caches, so the re-reads are
    not HBM traffic; they are reported separately). Flops: both streams, QK
    and PV over each query's visible keys at 2 flops per multiply-add (the
    memory stream in its own windows, the prediction stream in Bk-key
    blocks; causal attention counts the same pairs whatever the window). The roofline is the one the intensity selects (MFMA for these
    shapes).
    """
    import numpy as np
    import torch

    from causal_streaming_decoding_amd.dual_stream import DualStreamAttention

    dev = "cuda:0"
    S, N, Hq, Hkv, D, theta = 4, 4096, 32, 8, 128, 1e6
    g = torch.Generator(device=dev).manual_seed(0)
    r = lambda h: torch.randn((S, N, h, D), generator=g, device=dev).to(torch.bfloat16)
    qm, km, vm, qp, kp, vp = r(Hq), r(Hkv), r(Hkv), r(Hq), r(Hkv), r(Hkv)
    filled = (torch.rand((S, N), generator=g, device=dev) < 0.5).to(torch.uint8)
    hev = HipEvents(torch.cuda.current_stream().cuda_stream)
    for kernel, Bk in [(kn, b) for kn in ("block", "window") for b in (16, 32, 64)]:
        ds = DualStreamAttention(S, N, Bk, Hq, Hkv, D, theta, torch.bfloat16, dev, kernel=kernel)
        ev = [(hev.create(), hev.create()) for _ in range(23)]
        for a_, b_ in ev:
            hev.record(a_)
            ds.forward(qm, km, vm, qp, kp, vp, filled)
            hev.record(b_)
        torch.cuda.synchronize()
        us = np.array([hev.elapsed_ms(a_, b_) for a_, b_ in ev[3:]]) * 1e3
        hev.destroy()
        row = Hkv * D * 2                                   # bytes of one position's k (or v)
        # every window reads its prefix's k and v once
        prefix_keys = lambda w: sum(j * w for j in range(N // w))
        prefix_reads = S * (prefix_keys(ds.memory_window) + prefix_keys(Bk)) * 2 * row
        byts = 2 * S * N * (Hq * D * 2 * 2 + 2 * row) + 2 * S * N * 2 * row
        # (query, visible key) pairs of one head: block j of w queries sees the
        # j*w keys before it and, causally, (w + 1) / 2 of its own on average
        pairs = lambda w: sum(w * (j * w + (w + 1) / 2) for j in range(N // w))
        flops = 4 * S * Hq * D * (pairs(ds.memory_window) + pairs(Bk))
        med = float(np.median(us))
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        if flops / byts < ridge:
            roof = {"bound": "hbm", "achieved": byts / (med * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": flops / (med * 1e-6) / 1e12,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = None
        line = {
            "workload": f"dual_stream_S{S}_N{N}_Bk{Bk}_qwen3_8b_heads",
            "kernel": {"block": "wedlm_block_attn_rope",
                       "window": "wedlm_window_attn_rope"}[kernel],
            "metric": "dual-stream attention forward latency", "unit": "us", "dtype": "bf16",
            "us": {"median": med, "p10": float(np.percentile(us, 10)),
                   "p90": float(np.percentile(us, 90))},
            "tokens_per_s": 2 * S * N / (med * 1e-6),
            "algorithmic_bytes": int(byts), "prefix_rereads_bytes": int(prefix_reads),
            "flops": flops, "intensity_flop_per_byte": flops / byts,
            "roofline": roof,
            "tflops_at_median": flops / (med * 1e-6) / 1e12,
            "data": "synthetic",
        }
        print(json.dumps(line), flush=True)
        del ds
        torch.cuda.empty_cache()


def read_bandwidth(args):
    """Achievable HBM read rate on this GPU (one JSON line): the library's read
    probe over 8 GiB as a plain stream and as 4 KB blocks in a random order,
    each at several grid sizes (best reported), plus a torch device copy."""
    import torch

    from causal_streaming_decoding_amd import wedlm as Wd

    dev = "cuda:0"
    nbytes = 8 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    n_blk = nbytes // 4096
    gen = torch.Generator(device="cpu").manual_seed(0)
    order = torch.randperm(n_blk, generator=gen).to(torch.int32).to(dev)
    grids = (1024, 2048, 4096, 8192)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    reps = 10

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    by_grid = {}
    for kind, blocks in (("stream", None), ("paged_4k", order)):
        for grid in grids:
            t = timed(lambda: Wd.wedlm_read_probe(src, nbytes, blocks, n_blk, sink, grid))
            by_grid[f"{kind}_grid{grid}"] = nbytes / t / 1e9
    half = nbytes // 2
    a, b = src[:half], torch.empty(half, dtype=torch.uint8, device=dev)
    t_copy = timed(lambda: b.copy_(a))
    best = {k: max(v for g, v in by_grid.items() if g.startswith(k + "_")) for k in
            ("stream", "paged_4k")}
    print(json.dumps({
        "metric": "achievable HBM read GB/s (probe)", "bytes": nbytes,
        "stream_read_gbps": best["stream"], "paged_4k_read_gbps": best["paged_4k"],
        "copy_read_plus_write_gbps": 2 * half / t_copy / 1e9,
        "peak_gbps": HBM_PEAK_GBPS, "stream_frac": best["stream"] / HBM_PEAK_GBPS,
        "paged_4k_frac": best["paged_4k"] / HBM_PEAK_GBPS,
        "by_grid": by_grid}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        config_latencies(args)
        return
    if args.lm_head:
        lm_head_latencies(args)
        return
    if args.decode_modes:
        decode_modes(args)
        return
    if args.dual_stream:
        dual_stream_latencies(args)
        return
    if args.read_bw:
        read_bandwidth(args)
        return

    import numpy as np
    import torch

    from causal_streaming_decoding_amd import workloads as WL
    from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
    from causal_streaming_decoding_amd.synth import make_step_inputs, stream_step_inputs, to_f64

    wl = WL.BY_NAME[args.workload]
    dev = "cuda:0"
    K, Wm = args.steps, args.warmup
    n_inputs = max(K, Wm, 1)
    print(f"[bench] {wl.name}: building inputs ({n_inputs} steps)", file=sys.stderr, flush=True)
    inp = make_step_inputs(wl, steps=n_inputs)
    st, _, _, _, _, L0 = upload_step_inputs(wl, inp, dev)
    step = make_window_step(wl, inp, dev, L0 + wl.W * n_inputs, fused_tail=not args.separate_tail)
    if args.overlap and not args.separate_tail:
        step.set_overlap(torch.cuda.Stream())
    step.fuse_entropy = step.fuse_entropy and not (args.separate_entropy or args.overlap or
                                                   args.separate_tail)
    ins = [stream_step_inputs(wl, s, dev) for s in range(n_inputs)]
    commit_log = torch.zeros((n_inputs, wl.B), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    snap = st.snapshot()

    print(f"[bench] warmup {Wm} steps", file=sys.stderr, flush=True)
    for s in range(Wm):
        q, k, v, logits = ins[s]
        step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s, commit_len=commit_log[s])
    torch.cuda.synchronize()
    # the library launches on the stream it is given; None is the null stream,
    # which is torch's current stream here
    hev = HipEvents(torch.cuda.current_stream().cuda_stream)
    labels = ("attn_start", "attn_end", "entropy_end")
    # the kernels are timed on a uniform sample of the steps: each event
    # record costs GPU idle time, which would otherwise be part of every step
    every = max(args.event_every, 1)
    sampled = list(range(0, K, every))
    reps = max(args.reps, 1)
    elapsed_reps, attn_ms, ent_ms, commits_reps = [], [], [], []
    for r in range(reps):
        st.restore(snap)
        commit_log.zero_()
        ev = {s: {lab: hev.create() for lab in labels} for s in sampled}
        torch.cuda.synchronize()
        print(f"[bench] timing {K} steps (repetition {r + 1} of {reps})", file=sys.stderr,
              flush=True)
        t0 = time.perf_counter()
        for s in range(K):
            q, k, v, logits = ins[s % n_inputs]
            mark = (lambda lab, e=ev[s]: hev.record(e[lab])) if s in ev else None
            step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s, commit_len=commit_log[s],
                     mark=mark)
        torch.cuda.synchronize()
        elapsed_reps.append(time.perf_counter() - t0)
        attn_ms += [hev.elapsed_ms(ev[s]["attn_start"], ev[s]["attn_end"]) for s in sampled]
        ent_ms += [hev.elapsed_ms(ev[s]["attn_end"], ev[s]["entropy_end"]) for s in sampled]
        hev.destroy()
        commits_reps.append(commit_log[:K].cpu().numpy().astype(np.int64))
    for c in commits_reps[1:]:
        if not np.array_equal(c, commits_reps[0]):
            raise RuntimeError("repetitions from the same state committed different tokens")
    elapsed = float(np.median(elapsed_reps))
    attn_ms = np.array(attn_ms)
    ent_ms = np.array(ent_ms)
    commits = commits_reps[0]

    # untimed replay of the same steps for the logits' entropy regime
    st.restore(snap)
    ent_all, score_all, filled_all = [], [], []
    for s in range(K):
        q, k, v, logits = ins[s % n_inputs]
        filled_all.append(st.filled.cpu().numpy().astype(bool))
        step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s)
        ent_all.append(step.entropy.cpu().numpy())
        score_all.append(step.score.cpu().numpy())
    ent_hist = entropy_report(np.stack(ent_all), np.stack(filled_all), np.stack(score_all), wl.tau)

    L = np.asarray(inp["prefix_len"], np.int64).copy()
    tot = {"kv": 0, "window": 0, "attn_out": 0, "commit": 0, "logits": 0}
    attn_bytes = ent_bytes = 0    # over the sampled steps of one repetition
    attn_bytes_all = 0            # over every timed step (as the byte counters see them)
    for s in range(K):
        b = step_bytes(wl, L, commits[s])
        for key in tot:
            tot[key] += b[key]
        a = b["kv"] + b["window"] + b["attn_out"] + b["commit"]
        if step.fuse_entropy:
            a += b["logits"]  # the launch also reads every logit once
        attn_bytes_all += a
        if s in sampled:
            attn_bytes += a
            ent_bytes += 0 if step.fuse_entropy else b["logits"]
        L += commits[s]
    attn_bytes *= reps  # the event samples of every repetition
    ent_bytes *= reps
    total_bytes = sum(tot.values())
    committed = int(commits.sum())
    attn_gbps = attn_bytes / (attn_ms.sum() * 1e-3) / 1e9
    # with the chunk pass in the attention's launch the second interval is the
    # tail alone (selection, state commit, next reorder)
    ent_gbps = ent_bytes / (ent_ms.sum() * 1e-3) / 1e9 if ent_bytes else None
    both_gbps = (attn_bytes + ent_bytes) / ((attn_ms.sum() + ent_ms.sum()) * 1e-3) / 1e9
    step_gbps = total_bytes / elapsed / 1e9
    alg_per_launch = attn_bytes / (len(sampled) * reps)

    if args.calibrate_copy:
        a = torch.empty(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    from causal_streaming_decoding_amd.profiling import read_traffic
    ratio = read_traffic(os.path.join(ROOT, "profiles", TRAFFIC_RECORD), wl.name)
    # counted bytes per launch = the recorded counted / algorithmic ratio times
    # this run's algorithmic bytes per launch (null once the kernel changed)
    traffic = None if ratio is None else ratio * alg_per_launch

    cpu = None
    if args.cpu_baseline_steps > 0:
        n = min(args.cpu_baseline_steps, n_inputs)
        print(f"[bench] cpu baseline: oracle on {n} steps", file=sys.stderr, flush=True)
        host_steps = [tuple(to_f64(t) for t in ins[s]) for s in range(n)]
        cpu = cpu_baseline(wl, inp, host_steps)

    result = {
        "metric": "window-steps/s + committed tokens/s; KV+logits HBM GB/s as % of peak",
        "value": K / elapsed,
        "unit": "window-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n_layers": wl.n_layers, "batch": wl.B, "q_heads": wl.Hq,
                   "kv_heads": wl.Hkv, "head_dim": wl.D, "window": wl.W, "vocab": wl.V,
                   "initial_prefix": int(L0), "page_size": wl.page_size,
                   "step_tail": "separate" if args.separate_tail else "fused",
                   "entropy_stream": ("side" if (args.overlap and not args.separate_tail) else
                                      "attention launch" if step.fuse_entropy else "same"),
                   "parallelism": "single GPU"},
        "timing": f"median of {reps} repetitions of steps 0..{K - 1} from the start state "
                  f"(window-steps/s per repetition: "
                  f"{', '.join(f'{K / e:.1f}' for e in elapsed_reps)})",
        "committed_tokens": committed,
        "committed_tokens_per_s": committed / elapsed,
        "step_hbm_gbps": step_gbps,
        "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "attn_plus_entropy_hbm_gbps": both_gbps,
        "attn_plus_entropy_hbm_frac": both_gbps / HBM_PEAK_GBPS,
        "entropy_hbm_gbps": ent_gbps,
        "bytes_per_step_avg": {k_: v_ / K for k_, v_ in tot.items()},
        "entropy_histogram": ent_hist,
        "roofline": {"kernel": "k_window_attn_bf16" + (" (carrying the entropy chunk pass)"
                                                        if step.fuse_entropy else ""),
                     "bound": "hbm", "achieved": attn_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": attn_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "traffic_over_algorithmic": ratio,
                     "avg_launch_ms": float(attn_ms.mean()),
                     "algorithmic_bytes_per_launch": alg_per_launch,
                     "algorithmic_bytes_per_launch_all_steps": attn_bytes_all / K,
                     "timed_launches": f"{len(sampled)} of {K} (every {every}th step) in each "
                                       f"of {reps} repetitions"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
